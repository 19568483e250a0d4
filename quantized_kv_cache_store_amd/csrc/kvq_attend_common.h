// Pieces shared by the decode and prefill attention kernels: the argument block,
// row geometry, f32 window partial, and host-side argument handling.
#pragma once

#include "kvq_internal.h"

namespace kvq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define KVQ_LOG2E 1.4426950408889634f

// The decode's run length for grids that take several rounds of resident blocks, chosen per call from
// the rows' lengths (on the device by the kernels, on the host by kvq_decode_split_lengths, with the
// same function): runs of k half chunks, k = 8, 4, 3 (4, 2 and 1.5 chunks), each block four runs.  The
// cost of k counts whole rounds of blocks, ceil(blocks(k) / slots), times a wave's time in steps,
// kRunStartSteps of start-up (query load and preparation, first ring loads: measured at about four
// steps) plus its run's 32-token steps.  A ragged batch's last round is then filled by shorter runs
// where that pays, while a uniform batch keeps its longest runs.  The host enables it only where every
// count below fits 32 bits and chunk_tokens is a power of two.
struct RunSplit {
  int on;           // 1: the run length comes from run_span; 0: AttendArgs::span
  int units;        // blocks per chunk group: kv heads x row tiles
  int slots;        // blocks resident at once: CUs x blocks per CU
  int half_chunk;   // chunk_tokens / 2
  int unit_shift;   // log2 of u = 2 chunk_tokens, the tokens of a block of k = 1
  int batch;
};
constexpr int kRunStartSteps = 4;
constexpr int kRunShortest = 3;   // the shortest candidate, in half chunks (the grid is sized for it)

template <class Len>
__host__ __device__ inline int run_span(const RunSplit& r, int n_recent, Len len) {
  // a block of runs of k half chunks covers k u tokens, so a row of Sq quantised tokens takes
  // ceil(Sq / (k u)) = ceil(ceil(Sq / u) / k) blocks; lengths are read 16 at a time (index clamped)
  // so that their loads are in flight together
  const unsigned um = (1u << r.unit_shift) - 1u;
  unsigned g8 = 0, g4 = 0, g3 = 0;
  for (int b0 = 0; b0 < r.batch; b0 += 16) {
    int S[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) S[k] = len(b0 + k < r.batch ? b0 + k : r.batch - 1);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int Sq = n_recent > 0 ? (S[k] > n_recent ? S[k] - n_recent : 0) : S[k];
      const unsigned q = b0 + k < r.batch ? ((unsigned)Sq + um) >> r.unit_shift : 0u;
      g8 += (q + 7u) >> 3;
      g4 += (q + 3u) >> 2;
      g3 += (q + 2u) / 3u;
    }
  }
  const int ks[3] = {8, 4, kRunShortest};
  const unsigned gs[3] = {g8, g4, g3};
  int best = 8;
  unsigned long long best_cost = 0;
  for (int i = 0; i < 3; ++i) {
    const unsigned blocks = gs[i] * (unsigned)r.units;
    const unsigned rounds = (blocks + (unsigned)r.slots - 1u) / (unsigned)r.slots;
    const unsigned long long cost = (unsigned long long)rounds * (32u * kRunStartSteps + (unsigned)ks[i] * r.half_chunk);
    if (i == 0 || cost < best_cost) {
      best_cost = cost;
      best = ks[i];
    }
  }
  return best * r.half_chunk;
}

struct AttendArgs {
  const uint8_t* kp;
  const uint8_t* vp;
  const uint8_t* ks;
  const uint8_t* vs;
  const float* kring;
  const float* vring;
  const float* q;
  float* ws;
  const int32_t* block_table;
  const int32_t* seq_len;
  const int32_t* q_start;   // [batch] position of query 0 (causal prefill), else null
  const float* qrot;        // prepared rows (prefill): f32 query, rotated for HAD, [rows][D], else null
  const int8_t* q8p;        // prepared rows: int8 query [rows][D]
  const float* sqp;         // prepared rows: its scale [rows]
  const int* qsump;         // prepared rows: sum of q8 per 32-element block [rows][D / 32]
  const float* kchunk;      // full-precision prefill: the chunk's own K rows f32 [batch][n_q][Hkv][D] (rotated
  const float* vchunk;      //   for HAD) and V rows, read as exact rows at positions seq_len[b] + i; else null
  int32_t* dbg;
  int Hkv, Hq, G, page_shift, n_recent, max_pages, chunk, nc1, max_seq_len;
  int nwin;      // partial slots of the f32 rows, the last nwin of a row's nc1 (full-precision prefill: one
                 // per slice of its f32 rows; else 1)
  int slice;     // full-precision prefill: f32 rows per slice (a multiple of 16)
  int nwg;       // prefill: groups of f32 rows at the end of the prefill kernel's grid (0: none, or their
                 // own launch)
  int n_q;       // queries per batch row (1 for decode)
  int batch;     // batch rows (decode: the grid is one-dimensional)
  int ngroups;   // blocks per row tile along the sequence: chunk groups of four, + 1 for the window
  int span;      // tokens each wave of the decode kernel streams (a multiple of 32; chunk elsewhere); with
                 // rs.on the shortest run the call may take (it sizes the grid and the partial slots)
  RunSplit rs;   // decode: the run length chosen from the rows' lengths, for grids of several rounds
  int causal;    // rows see t <= q_start + i
  int skip;      // causal skip: stop streaming past the tile's last visible token
  float alpha;
};

// Row R of (b, hk) is query i = R / G of head hk * G + R % G; its flat index in
// [batch][n_q][Hq] addresses q, out and (times the chunk count) the partials.
__device__ __forceinline__ size_t row_index(const AttendArgs& a, int b, int hk, int R) {
  const int i = R / a.G;
  return ((size_t)b * a.n_q + i) * a.Hq + hk * a.G + (R - i * a.G);
}

// Last visible position of row R (rows past the tile's valid count see nothing).
__device__ __forceinline__ int row_limit(const AttendArgs& a, int qs0, int R, int nrows) {
  if (R >= nrows) return -1;
  return a.causal ? qs0 + R / a.G : 0x7fffffff;
}

// Reductions over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48), on the VALU:
// v_permlane16_swap / v_permlane32_swap applied to two copies of a value leave in the two
// registers the value of the lane and of its partner row, in row order, so both lanes of a pair
// compute the same result.  Written as inline assembly with both registers read-write (the
// compiler's built-in for it folds its two results into one), with the wait states the swap
// needs after the VALU writes of its operands.
__device__ __forceinline__ void row_pair(float v, int swap32, float& lo, float& hi) {
  float x = v, y = v;
  if (swap32)
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  else
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  lo = x;
  hi = y;
}

__device__ __forceinline__ float max_over_rows(float v) {
  float a, b;
  row_pair(v, 0, a, b);
  row_pair(fmax_nc(a, b), 1, a, b);
  return fmax_nc(a, b);
}

__device__ __forceinline__ float sum_over_rows(float v) {
  float a, b;
  row_pair(v, 0, a, b);
  row_pair(a + b, 1, a, b);
  return a + b;
}

// The Hadamard layout keeps one f32 V scale per token, which the f16 P V product cannot carry at
// every magnitude.  A wave keeps e, the binary exponent of the largest V scale it has seen
// (s = m * 2^e with m in [0.5, 1), v_frexp_exp), and feeds the f16 P operand p * s / 2^e, which lies in
// [0, 1] for every token so far; its accumulators are in units of 2^e, rescaled (exactly, by a power of
// two) when e grows, and multiplied by 2^e in f32 when the partial is written.  The operands, and so
// the accumulated bits, are the same for V scaled by any power of two.  kNoExp: nothing seen yet.
constexpr int kNoExp = -(1 << 20);
__device__ __forceinline__ int vscale_exp(float vmax) {
  return vmax > 0.0f ? __builtin_amdgcn_frexp_expf(vmax) : kNoExp;
}

__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// Narrow partial records (narrow_stride): x = frexp exponent of the row's largest |o| (0 when every
// o is 0), h = o * 2^(15 - x) rounded to f16 (|h| < 2^15, exact scaling by ldexp), and the record's
// exponent x - 15 plus the accumulators' own unit.
__device__ __forceinline__ int narrow_exp(float amax) { return __builtin_amdgcn_frexp_expf(amax); }
__device__ __forceinline__ uint32_t narrow_pk(float a, float b, int x) {
  return as_u32(h2{(_Float16)__builtin_amdgcn_ldexpf(a, 15 - x), (_Float16)__builtin_amdgcn_ldexpf(b, 15 - x)});
}

// q6_0 octet (low-nibble dword + 16 bits of top-bit pairs) -> biased 6-bit codes
// (code + 32) as bytes, even elements [0,2,4,6] in `ev`, odd [1,3,5,7] in `od`.
__device__ __forceinline__ void q6_octet(uint32_t lo, uint32_t hi16, uint32_t& ev, uint32_t& od) {
  const uint32_t w = __builtin_amdgcn_perm(hi16, hi16, 0x01010000u);   // bytes [b0, b0, b1, b1]
  const uint32_t te = ((w << 4) & 0x00300030u) | (w & 0x30003000u);
  const uint32_t to = ((w << 2) & 0x00300030u) | ((w >> 2) & 0x30003000u);
  ev = ((lo & 0x0F0F0F0Fu) | te) ^ 0x20202020u;
  od = (((lo >> 4) & 0x0F0F0F0Fu) | to) ^ 0x20202020u;
}

// Reductions over the 16 lanes of a row of the wave (lanes 16 k .. 16 k + 15): DPP rotations
// within the row by 1, 2, 4, 8 leave every lane with the reduction of all 16.
__device__ __forceinline__ float row16_rot(float v, int n) {
  const int x = __builtin_bit_cast(int, v);
  int y;
  switch (n) {
    case 1: y = __builtin_amdgcn_update_dpp(0, x, 0x121, 0xF, 0xF, false); break;
    case 2: y = __builtin_amdgcn_update_dpp(0, x, 0x122, 0xF, 0xF, false); break;
    case 4: y = __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false); break;
    default: y = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false); break;
  }
  return __builtin_bit_cast(float, y);
}
// The maximum: each rotation is one DPP max (max of the rotated lane's value and the lane's own, never
// NaN), which also spares the quieting of the moved operand that fmaxf would add.  s_nop 1: the wait
// states a DPP read of a VGPR needs after a VALU wrote it.
__device__ __forceinline__ float row16_max(float v) {
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:1 row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:2 row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf" : "+v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf" : "+v"(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += row16_rot(v, 1);
  v += row16_rot(v, 2);
  v += row16_rot(v, 4);
  return v + row16_rot(v, 8);
}

// Butterflies between partner lane rows (lanes l and l ^ 16, or l and l ^ 32): row_pair leaves the
// lower row's value in lo and the upper row's in hi, so the lower lane takes lo + hi and the upper
// lo - hi, the (a, b) -> (a + b, a - b) of the transform with a the lower-index element.
__device__ __forceinline__ float butterfly_rows(float v, int swap32, bool upper) {
  float lo, hi;
  row_pair(v, swap32, lo, hi);
  return upper ? lo - hi : lo + hi;
}

// Query preparation of one row inside a wave, in the order the int8 MFMA's B operand takes: lane
// row r (lanes 16 r .. 16 r + 15 all hold the same row in their column) keeps elements
// 32 g + 8 r + i (i < 8) of every 32-element block g.  The arithmetic is that of the query
// preparation kernel, step for step: the Hadamard layout's butterflies with strides 1, 2, 4 inside
// the lane, 8 and 16 between lane rows, 32, 64, ... inside the lane again (the ascending stage order
// of the encoding), each in f32, then f32(1/sqrt(D)); amax over the row, sq = amax / 127 (IEEE
// division), q8 = rint(x / sq) clamped to [-127, 127]; per-block sums of q8.
//
// Float-query mode (FQ): the query also gets two more int8 terms, each the residual of the terms
// before it at 254 times their resolution: t1 = f32(f32(x / sq) - q8) * 254, r1 = rint(t1),
// r2 = rint(f32(t1 - r1) * 254), all within [-127, 127], so that sq * (q8 + r1 / 254 + r2 / 254^2)
// stands for x to within about sq / 129032 (f32 resolution at the vector's largest element).  The
// integer dot then runs three times on the same codes, and (254 I(q8) + I(r1)) * 254 + I(r2) is
// the block dot with that query (the bracket exact in i32, the rest one f32 rounding).
template <int D>
struct RowQ {
  long qB[D / 32];     // B operand of block g: codes [0, 2, 4, 6, 1, 3, 5, 7] of the lane's 8 (the order
                       // in which the A operand unpacks even and odd nibbles); the 8-bit layout, whose
                       // A operand is 8 stored bytes, takes them in element order [0 .. 7]
  int qsum[D / 32];    // sum of q8 over block g (every lane)
  long qBl[2 * (D / 32)];    // FQ: the residual terms r1 (blocks 0 .. NG - 1) and r2 (NG .. 2 NG - 1), same order
  int qsuml[2 * (D / 32)];   // FQ: their block sums
  float sq;
};

// The 8 codes c[0..7] of a lane as the B operand (element order for the 8-bit layout, else even then
// odd elements).
template <int L>
__device__ __forceinline__ long pack_b_operand(const int* c) {
  const int s1 = L == Q80 ? 1 : 2, s2 = L == Q80 ? 4 : 1;   // element of byte k of lo / hi: s1 * k (+ s2)
  const uint32_t lo = (uint32_t)(c[0] & 0xFF) | ((uint32_t)(c[s1] & 0xFF) << 8) |
                      ((uint32_t)(c[2 * s1] & 0xFF) << 16) | ((uint32_t)(c[3 * s1] & 0xFF) << 24);
  const uint32_t hi = (uint32_t)(c[s2] & 0xFF) | ((uint32_t)(c[s2 + s1] & 0xFF) << 8) |
                      ((uint32_t)(c[s2 + 2 * s1] & 0xFF) << 16) | ((uint32_t)(c[s2 + 3 * s1] & 0xFF) << 24);
  return __builtin_bit_cast(long, u32x2{lo, hi});
}

// The lane row's elements 32 g + 8 r .. 32 g + 8 r + 7 of every block g of a query row (loaded apart
// from the preparation, so that a kernel can issue other loads before it waits for these).
template <int D>
__device__ __forceinline__ void load_row_lanes(const float* qrow, int r, float (&x)[D / 32][8]) {
#pragma unroll
  for (int g = 0; g < D / 32; ++g) {
    const float4 u = *reinterpret_cast<const float4*>(qrow + 32 * g + 8 * r);
    const float4 w = *reinterpret_cast<const float4*>(qrow + 32 * g + 8 * r + 4);
    x[g][0] = u.x; x[g][1] = u.y; x[g][2] = u.z; x[g][3] = u.w;
    x[g][4] = w.x; x[g][5] = w.y; x[g][6] = w.z; x[g][7] = w.w;
  }
}

template <int L, int D, bool FQ = false>
__device__ __forceinline__ void prepare_row_lanes(float (&x)[D / 32][8], int r, RowQ<D>& out) {
#pragma clang fp contract(off)
  constexpr int NG = D / 32;
  if (L == HAD) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((i & h) == 0) {
            const float p = x[g][i], q = x[g][i + h];
            x[g][i] = p + q;
            x[g][i + h] = p - q;
          }
#pragma unroll
    for (int m = 0; m < 2; ++m)   // strides 8, 16: lane rows r ^ 1, r ^ 2
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[g][i] = butterfly_rows(x[g][i], m, (r >> m) & 1);
#pragma unroll
    for (int hg = 1; hg < NG; hg <<= 1)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        if ((g & hg) == 0)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float p = x[g][i], q = x[g + hg][i];
            x[g][i] = p + q;
            x[g + hg][i] = p - q;
          }
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[g][i] = x[g][i] * hadamard_norm<D>();
  }
  float m = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[g][i]));
  m = max_over_rows(m);
  const float s = m / 127.0f;
  out.sq = s;
  // The quotients x / s.  With r = 1 / s correctly rounded (one IEEE division per row), q0 = x r
  // lies within an ulp of x / s, the residual x - s q0 is exact (an fma), and q0 + (x - s q0) r
  // rounds to the correctly rounded quotient (Markstein's correction step) whenever that residual
  // does not underflow, which holds for |x| >= 2^-102.  Rows with s >= 2^-82 take this form: their
  // smaller elements have quotients below 2^-20, whose codes (all three terms of the float-query
  // mode) are zero whatever the quotient's last bits.  Rows below 2^-82 take the IEEE division.
  if (s >= 0x1p-82f) {
    const float rs = 1.0f / s;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q0 = x[g][i] * rs;
        x[g][i] = fmaf(fmaf(-s, q0, x[g][i]), rs, q0);
      }
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[g][i] = s != 0.0f ? x[g][i] / s : 0.0f;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    int c[8], cl[8], cm[8], sum = 0, suml = 0, summ = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = x[g][i];
      const float n = fminf(fmaxf(rintf(y), -127.0f), 127.0f);
      c[i] = (int)n;
      sum += c[i];
      if (FQ) {
        const float t1 = (y - n) * 254.0f;
        const float r1 = fminf(fmaxf(rintf(t1), -127.0f), 127.0f);
        cl[i] = (int)r1;
        suml += cl[i];
        cm[i] = (int)fminf(fmaxf(rintf((t1 - r1) * 254.0f), -127.0f), 127.0f);
        summ += cm[i];
      }
    }
    out.qB[g] = pack_b_operand<L>(c);
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    out.qsum[g] = sum;
    if (FQ) {
      out.qBl[g] = pack_b_operand<L>(cl);
      out.qBl[NG + g] = pack_b_operand<L>(cm);
      suml += __shfl_xor(suml, 16);
      suml += __shfl_xor(suml, 32);
      out.qsuml[g] = suml;
      summ += __shfl_xor(summ, 16);
      summ += __shfl_xor(summ, 32);
      out.qsuml[NG + g] = summ;
    }
  }
}

// The f32 query of a row rotated in a wave, for the window: lane row r holds the contiguous
// elements N r .. N r + N - 1 (N = D / 4): butterflies with strides below N inside the lane,
// N and 2 N between lane rows, then f32(1/sqrt(D)).
template <int D>
__device__ __forceinline__ void rotate_quarters(float* x, int r) {
#pragma clang fp contract(off)
  constexpr int N = D / 4;
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & h) == 0) {
        const float p = x[i], q = x[i + h];
        x[i] = p + q;
        x[i + h] = p - q;
      }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = butterfly_rows(x[i], m, (r >> m) & 1);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = x[i] * hadamard_norm<D>();
}

// Window partial: exact f32 rows of the newest W = min(S, n_recent) tokens (HAD: rotated basis),
// each row masked by its limit, on the f32 MFMA (v_mfma_f32_16x16x4f32).  One wave takes a tile
// of 16 rows and walks 16-token tiles k = k0, k0 + kstep, ... of the window with an online
// softmax:
//   * Q K^T as C[row][token] = sum_d Q[row][d] K[token][d]: lane (col, r) holds the query of row
//     col and K of token col for d = 32 r + i in MFMA i (i < D / 4), both from registers; C gives
//     lane (col, r) the scores of rows 4 r + j, token col (a row's 16 tokens are a 16-lane row);
//   * P V as C[row][d] += sum_t P[row][t] V[t][d], four tokens per MFMA: the A operand (lane
//     (col, r): P[row col][token 4 q + r]) is P transposed through LDS, the B operand (lane
//     (col, r): V[token 4 q + r][d]) comes from the V tile staged in LDS.  The output rows 4 r + j
//     are the rows of the lane's scores, so the online rescale is lane-local.
// The wave's LDS: the V tile [16][D + 16] f32, rows padded (conflict-free B reads), and P in the
// padding: P[row R][token T] at [T][D + (R ^ ((T >> 2) & 3))], which both the writes (lanes: 16
// tokens x rows 4 r + j) and the transposing reads (lanes: 16 rows x tokens 4 qq + r) spread over
// all 64 banks, since a padded row starts 16 banks after the previous one.
// Tiles past the farthest limit of the wave's rows are not visited: a wholly masked tile would
// leave m, l and o exactly as they are.  (The prefill's f32 rows, which also include a chunk's own
// rows, go through f32_rows_block, which stages each tile once for a block's four waves.)
template <int D>
__host__ __device__ constexpr int window_wave_lds() { return 16 * (D + 16) * 4; }
template <int D>
__host__ __device__ constexpr int window_lds_bytes() { return 4 * window_wave_lds<D>(); }

template <int D>
struct WinState {
  v4f o[D / 16];     // rows 4 r + j, d = 16 dt + col
  float m[4], l[4];  // per row 4 r + j (l: this lane's part, summed over the row at the end)
};

template <int L, int D>
__device__ __forceinline__ void window_wave(const AttendArgs& a, float* vt, int b, int hk, int S, int row0, int nvalid,
                                            int qs0, int k0, int kstep, int lane, WinState<D>& st) {
  constexpr int NI = D / 4;           // MFMAs of Q K^T (d = 32 r + i... four lanes groups of D / 4)
  constexpr int VS = D + 16;          // V tile row stride (floats)
  const int col = lane & 15, r = lane >> 4;
  const int nrows = a.n_q * a.G;
  const int W = min(S, a.n_recent);
  const int w0 = S - W;
  const int NT = W;
  const size_t ring0 = ((size_t)b * a.Hkv + hk) * a.n_recent;
  const float cl = a.alpha * KVQ_LOG2E;
  // the query of row col (prepared rows: rotated for HAD), elements NI r .. NI r + NI - 1
  float q[NI];
  {
    const float* qsrc = a.qrot ? a.qrot : a.q;   // prepared rows (prefill: rotated for HAD) or the raw query
    const bool ok = col < nvalid;
    const float* qr = qsrc + (ok ? row_index(a, b, hk, row0 + col) * D : 0) + NI * r;
#pragma unroll
    for (int i = 0; i < NI; i += 4) {
      const float4 v = ok ? *reinterpret_cast<const float4*>(qr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      q[i] = v.x;
      q[i + 1] = v.y;
      q[i + 2] = v.z;
      q[i + 3] = v.w;
    }
    if (L == HAD && !a.qrot) rotate_quarters<D>(q, r);
  }
  int lim[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) lim[j] = 4 * r + j < nvalid ? row_limit(a, qs0, row0 + 4 * r + j, nrows) : -1;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) st.o[i] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    st.m[j] = -INFINITY;
    st.l[j] = 0.0f;
  }
  int ntiles = (NT + 15) / 16;
  {
    const int lmax = nvalid > 0 ? row_limit(a, qs0, row0 + nvalid - 1, nrows) : -1;   // the tile's farthest limit
    if (lmax < w0) ntiles = 0;
    else if ((lmax - w0) / 16 + 1 < ntiles) ntiles = (lmax - w0) / 16 + 1;
  }
  for (int k = k0; k < ntiles; k += kstep) {
    const int t0 = 16 * k;
    const int t = t0 + col;
    const bool tok_ok = t < NT;
    int slot = w0 + (tok_ok ? t : 0);
    slot -= (slot / a.n_recent) * a.n_recent;
    const size_t ro = (ring0 + (size_t)slot) * D + NI * r;
    const float* ksrc = a.kring + ro;
    const float* vsrc = a.vring + ro;
    // ---- Q K^T
    v4f c = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; i += 4) {
      const float4 kv = tok_ok ? *reinterpret_cast<const float4*>(ksrc + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(q[i], kv.x, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(q[i + 1], kv.y, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(q[i + 2], kv.z, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(q[i + 3], kv.w, c, 0, 0, 0);
    }
    // ---- V tile to LDS (token col, elements NI r ..), zeros past the last token
#pragma unroll
    for (int i = 0; i < NI; i += 4) {
      const float4 vv = tok_ok ? *reinterpret_cast<const float4*>(vsrc + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(vt + col * VS + NI * r + i) = vv;
    }
    // ---- online softmax of rows 4 r + j over the tile's 16 tokens (lanes of the 16-lane row)
    float p[4], corr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = (tok_ok && w0 + t <= lim[j]) ? c[j] * cl : -INFINITY;
      const float m_new = fmax_nc(st.m[j], row16_max(x));
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;   // a row that sees nothing yet: p = 0
      corr[j] = __builtin_amdgcn_exp2f(st.m[j] - m_use);   // results below 2^-126 (against a maximum of 1)
      p[j] = __builtin_amdgcn_exp2f(x - m_use);            // may flush: they change no sum
      st.l[j] = st.l[j] * corr[j] + p[j];
      st.m[j] = m_new;
      vt[col * VS + D + ((4 * r + j) ^ (col >> 2))] = p[j];   // P[row 4 r + j][token col]
    }
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      v4f o = st.o[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] *= corr[j];
      st.o[i] = o;
    }
    // ---- P V
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float pa = vt[(4 * qq + r) * VS + D + (col ^ qq)];   // P[row col][token 4 qq + r]
      const float* vrow = vt + (4 * qq + r) * VS + col;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, vrow[16 * dt], st.o[dt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) st.l[j] = row16_sum(st.l[j]);
}

// Write a window state as the (narrow) partial of rows row0 + 4 r + j (< nvalid) in partial slot
// `slot` (prefill).  Lane col holds o[16 dt + col]; lane pairs (col, col ^ 1) swap one value so that
// each writes a dword of two neighbouring elements: the even lane o[16 dt + col], o[16 dt + col + 1]
// for even dt, the odd lane the pair at col - 1 for odd dt.
template <int D>
__device__ __forceinline__ void window_store(const AttendArgs& a, const WinState<D>& st, int b, int hk, int row0, int nvalid,
                                             int lane, int slot) {
  const int col = lane & 15, r = lane >> 4;
  const bool odd = (col & 1) != 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float amax = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) amax = fmax_pos(amax, fabsf(st.o[dt][j]));
    const int x = narrow_exp(row16_max(amax));
    uint32_t pk[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 16; dt += 2) {
      // even lane: keeps o[dt] (its own element 16 dt + col), sends o[dt + 1]; odd lane the reverse
      const float keep = odd ? st.o[dt + 1][j] : st.o[dt][j];
      const float send = odd ? st.o[dt][j] : st.o[dt + 1][j];
      const float got = __shfl_xor(send, 1);
      pk[dt / 2] = odd ? narrow_pk(got, keep, x) : narrow_pk(keep, got, x);
    }
    if (4 * r + j >= nvalid) continue;
    float* dst = a.ws + (row_index(a, b, hk, row0 + 4 * r + j) * a.nc1 + slot) * narrow_stride(D);
    uint32_t* hw = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
    for (int dt = 0; dt < D / 16; dt += 2) hw[8 * (dt + (odd ? 1 : 0)) + (col >> 1)] = pk[dt / 2];
    if (col == 0) {
      dst[D / 2] = st.m[j];
      dst[D / 2 + 1] = st.l[j];
      reinterpret_cast<int*>(dst)[D / 2 + 2] = x - 15;
    }
  }
}

// Window partial of one tile of at most 16 rows by the block's four waves, which split the
// window's 16-token tiles (wave w: tiles w, w + 4, ...) and merge their states through LDS in a
// fixed order (decode).
template <int L, int D>
__device__ __forceinline__ void window_tile_block(const AttendArgs& a, unsigned char* smem, int b, int hk, int S, int row0,
                                                  int nvalid, int qs0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  WinState<D> st;
  window_wave<L, D>(a, reinterpret_cast<float*>(smem + wave * window_wave_lds<D>()), b, hk, S, row0, nvalid, qs0, wave, 4,
                    lane, st);
  __syncthreads();
  // each wave's state as [16 rows][D + 4] (o, m, l)
  constexpr int PST = D + 4;
  float* mo = reinterpret_cast<float*>(smem) + wave * 16 * PST;
  const int col = lane & 15, r = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float* dst = mo + (4 * r + j) * PST;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) dst[16 * dt + col] = st.o[dt][j];
    if (col == 0) {
      dst[D] = st.m[j];
      dst[D + 1] = st.l[j];
    }
  }
  __syncthreads();
  const int row = tid >> 4, e0 = (tid & 15) * (D / 16);   // 16 threads per row
  if (row < nvalid) {
    const float* src = reinterpret_cast<const float*>(smem) + row * PST;
    float mk[4], M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      mk[k] = src[k * 16 * PST + D];
      M = fmaxf(M, mk[k]);
    }
    float w[4], l = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w[k] = mk[k] == -INFINITY ? 0.0f : exp2f(mk[k] - M);
      l += w[k] * src[k * 16 * PST + D + 1];
    }
    float* dst = a.ws + (row_index(a, b, hk, row0 + row) * a.nc1 + (a.nc1 - 1)) * partial_stride(D);
#pragma unroll
    for (int e = 0; e < D / 16; ++e) {
      float o = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) o += w[k] * src[k * 16 * PST + e0 + e];
      dst[e0 + e] = o;
    }
    if ((tid & 15) == 0) {
      dst[D] = M;
      dst[D + 1] = l;
    }
  }
}

// ----------------------------------------------------------------------------- staging of 32-token steps

// Staging of one 32-token step in a wave's LDS slice.  Two ways to fill it:
//   * register ring (DMA = false): 16-byte loads into registers several steps ahead, then one
//     copy per step to [K payload rows 32 x RS][V payload rows 32 x RS][K records 32 x SB]
//     [V records 32 x SB]; payload rows are padded to RS = PB + 16 bytes, which spreads the reads
//     of a 16-row column (K: one dword per lane from 16 rows; V: 16 dwords of one row times four
//     rows 4 apart) over all 64 LDS banks.
//   * direct loads (DMA = true): global_load_lds_dwordx4 writes the step straight into a K slot
//     [K payload 32 x PB][K records 32 x SB] and a V slot [V payload][V records] of LDS rings,
//     1 KiB per instruction (lane i's 16 bytes at slot offset + 16 i), so no
//     registers hold data in flight.  Rows cannot be padded then; for 64-byte rows the chunks are
//     placed instead so that the same reads stay conflict-free: K chunk c of row t goes to chunk
//     position c ^ ((t >> 2) & 3) of row t, and V row t to row position vperm(t), which swaps the
//     two 2-bit fields of t within its 16-row half (rows 4 apart then land 16 banks apart).
//     The 8-bit layout's rows (D bytes, CPR = D / 16 chunks) are read 8 bytes per lane: K chunk c
//     of row t goes to position c ^ kswz8(t) of its row (the 16 rows of an operand then fill every
//     bank twice), and V chunk j of the slot (j = CPR t + c) to j ^ (8 ((t >> 2) & 1)) (rows 4
//     apart, read together, alternate between the two halves of the banks).
template <int L, int D, bool DMA = false>
struct Step {
  using T = Layout<L, D>;
  static constexpr int PB = T::PB, SB = T::SB;
  static constexpr int RS = DMA ? PB : PB + 16;
  // K side offsets from the K base, V side offsets from the V base.  Register ring: one buffer,
  // both bases equal.  Direct loads: separate K and V slots of HALF bytes each.
  static constexpr int KP = 0, KR = DMA ? 32 * PB : 64 * RS;
  static constexpr int VP = DMA ? 0 : 32 * RS, VR = DMA ? 32 * PB : 64 * RS + 32 * SB;
  static constexpr int HALF = 32 * (PB + SB);
  static constexpr int BYTES = 64 * RS + 64 * SB;   // register ring buffer
  static constexpr bool SWZ = DMA && PB == 64;
  static constexpr bool SWZ8 = DMA && L == Q80;
  static constexpr int CPR = PB / 16;   // 16-byte chunks per row
  // register ring
  static constexpr int PAY_SLOTS = (2 * PB + 63) / 64;   // 16-byte chunks of 32 payload rows, per lane
  static constexpr int REC_SLOTS = (4 * SB + 63) / 64;   // K and V records together
  static constexpr int SLOTS = 2 * PAY_SLOTS + REC_SLOTS;
  // direct loads: K and V issued as separate groups, each the tensor's payload (PB / 32
  // instructions of 1 KiB) and its 32 records (one instruction per 16-token half)
  static constexpr int PAY_INSTR = PB / 32;
  static constexpr int GROUP = PAY_INSTR + 2;
  static_assert(SB <= 64, "one record instruction per half");

  __device__ static int vperm(int t) { return (t & 16) | ((t & 3) << 2) | ((t >> 2) & 3); }
  // byte offset of dword r of the 16-byte code block g of K row t (layouts with 4-bit codes)
  __device__ static int kword(int t, int g, int r) {
    return SWZ ? KP + 16 * (4 * t + (g ^ ((t >> 2) & 3))) + 4 * r : KP + t * RS + 4 * (4 * g + r);
  }
  // byte offset of dword oc of V row t (layouts with 4-bit codes)
  __device__ static int vword(int t, int oc) {
    return SWZ ? VP + 16 * (4 * vperm(t) + (oc >> 2)) + 4 * (oc & 3) : VP + t * RS + 4 * oc;
  }
  // 8-bit layout: chunk placement (both maps are their own inverses)
  __device__ static int kswz8(int t) { return 2 * ((t >> 1) & (CPR / 2 - 1)); }
  __device__ static int vlin8(int j) { return j ^ (8 * (((j / CPR) >> 2) & 1)); }
  // byte offset of the 8 codes 32 g + 8 r .. 32 g + 8 r + 7 of K row t (8-bit layout)
  __device__ static int kbytes8(int t, int g, int r) {
    const int c = 2 * g + (r >> 1);
    return SWZ8 ? KP + t * PB + 16 * (c ^ kswz8(t)) + 8 * (r & 1) : KP + t * RS + 32 * g + 8 * r;
  }
  // byte offset of the 8 codes of octet oc (elements 8 oc .. 8 oc + 7) of V row t (8-bit layout)
  __device__ static int vbytes8(int t, int oc) {
    return SWZ8 ? VP + 16 * vlin8(t * CPR + (oc >> 1)) + 8 * (oc & 1) : VP + t * RS + 8 * oc;
  }
};

// Physical row indices of the two 16-token halves of the step at T (wave-uniform).
struct HalfRows {
  size_t r0, r1;
};

// The same rows from page entries read through the scalar cache (the page index is wave-uniform):
// no vector registers hold the page list and no vector-memory counter is involved.
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;

__device__ __forceinline__ size_t page_row(const AttendArgs& a, int b, int hk, int t) {
  const const_i32_ptr bt = (const_i32_ptr)a.block_table;
  const int phys = bt[(size_t)b * a.max_pages + (t >> a.page_shift)];
  return (((size_t)phys * a.Hkv + hk) << a.page_shift) + (size_t)(t & ((1 << a.page_shift) - 1));
}

__device__ __forceinline__ HalfRows half_rows_s(const AttendArgs& a, int b, int hk, int T, int t_end) {
  HalfRows h;
  h.r0 = page_row(a, b, hk, T);   // T < t_end for every issued step
  h.r1 = T + 16 < t_end ? page_row(a, b, hk, T + 16) : h.r0;
  return h;
}

// One direct load to LDS: lane i's 16 bytes at `src` go to LDS byte address lds + 16 i (lds is
// wave-uniform and travels in m0).
__device__ __forceinline__ void dma16(const uint8_t* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" : : "v"(src), "{m0}"(lds) : "memory");
}

// Wait until at most N vector-memory operations of the wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// The same with a wave-uniform base address in SGPRs and a 32-bit lane offset.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}

// The K half (ISV = false: K payload and records) or the V half of a step's direct loads into
// the K or V slot at LDS address `slot`; ST::GROUP instructions.  An instruction whose 64 chunks lie
// in one 16-token half (rows contiguous in one page) takes that half's row address as a uniform
// base and a loop-invariant lane offset; the records go as one instruction per half.
template <class ST, bool ISV>
__device__ __forceinline__ void issue_dma_half(const AttendArgs& a, HalfRows hr, int lane, uint32_t slot) {
  constexpr int PB = ST::PB, SB = ST::SB, CPR = PB / 16;
  const uint8_t* const pay = ISV ? a.vp : a.kp;
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#pragma unroll
  for (int k = 0; k < ST::PAY_INSTR; ++k) {
    const int p = 64 * k + lane;
    int t, c;   // row and chunk that position p holds
    if (ST::SWZ) {
      t = ISV ? ST::vperm(p >> 2) : (p >> 2);
      c = ISV ? (p & 3) : ((p & 3) ^ ((t >> 2) & 3));
    } else if (ST::SWZ8) {
      const int j = ISV ? ST::vlin8(p) : p;
      t = j / CPR;
      c = ISV ? j - t * CPR : ((j - t * CPR) ^ ST::kswz8(t));
    } else {
      t = p / CPR;
      c = p - t * CPR;
    }
    const uint32_t lds = slot + (ISV ? ST::VP : ST::KP) + 1024 * k;
    const bool one_half = (64 * k) / (16 * CPR) == (64 * k + 63) / (16 * CPR);   // folded: k is unrolled
    if (one_half) {
      const int half = (64 * k) / (16 * CPR);
      dma16(pay + (half ? hr.r1 : hr.r0) * PB, (uint32_t)((t & 15) * PB + 16 * c), lds);
    } else {
      const size_t row = (t < 16 ? hr.r0 : hr.r1) + (size_t)(t & 15);
      dma16(pay + row * PB + 16 * c, lds);
    }
  }
  const uint8_t* const rec = ISV ? a.vs : a.ks;
  if (lane < SB) {   // 16 records of SB bytes per half: SB chunks of 16 bytes
#pragma unroll
    for (int h = 0; h < 2; ++h)
      dma16(rec + (h ? hr.r1 : hr.r0) * SB, (uint32_t)(16 * lane), slot + (ISV ? ST::VR : ST::KR) + 16 * SB * h);
  }
}

// ----------------------------------------------------------------------------- host side

static inline int chunks_of(int max_seq_len, int chunk) { return (max_seq_len + chunk - 1) / chunk; }

static inline kvq_status check_attend_args(const kvq_cache* c, const void* q, int32_t batch, int32_t Hq,
                                           const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                                           int32_t max_seq_len) {
  kvq_status st = validate_cache(c);
  if (st != KVQ_OK) return st;
  if (!q || !block_table || !seq_len) return fail(KVQ_ERR_INVALID_ARG, "q, block_table and seq_len must be non-null");
  if (batch < 1) return fail(KVQ_ERR_INVALID_ARG, "batch must be >= 1");
  if (Hq < 1 || Hq % c->num_kv_heads) return fail(KVQ_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (max_pages < 1 || (int64_t)max_pages * c->page_size < max_seq_len)
    return fail(KVQ_ERR_INVALID_ARG, "max_pages_per_seq * page_size must cover max_seq_len");
  if (c->n_recent > 512) return fail(KVQ_ERR_UNSUPPORTED, "n_recent above 512");
  return KVQ_OK;
}

// Argument block for a launch over rows of n_q queries; ngroups is set for the decode kernel
// (chunk groups of four, + 1 window group) and replaced by the prefill.
static inline AttendArgs make_args(const kvq_cache* c, const float* q, int32_t Hq, int32_t n_q, float alpha,
                                   const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                                   int32_t max_seq_len, int32_t chunk, void* workspace) {
  AttendArgs a;
  memset(&a, 0, sizeof(a));
  a.kp = (const uint8_t*)c->k_payload;
  a.vp = (const uint8_t*)c->v_payload;
  a.ks = (const uint8_t*)c->k_scale;
  a.vs = (const uint8_t*)c->v_scale;
  a.kring = c->k_recent;
  a.vring = c->v_recent;
  a.q = q;
  a.ws = (float*)workspace;
  a.block_table = block_table;
  a.seq_len = seq_len;
  a.Hkv = c->num_kv_heads;
  a.Hq = Hq;
  a.G = Hq / c->num_kv_heads;
  a.page_shift = __builtin_ctz((unsigned)c->page_size);
  a.n_recent = c->n_recent;
  a.max_pages = max_pages;
  a.chunk = chunk;
  const int nch = chunks_of(max_seq_len, chunk);
  a.nc1 = nch + 1;
  a.nwin = 1;
  a.max_seq_len = max_seq_len;
  a.n_q = n_q;
  a.ngroups = (nch + 3) / 4 + (c->n_recent > 0 ? 1 : 0);
  a.span = chunk;
  a.alpha = alpha;
  return a;
}

// Blocks along x of the decode kernel: row tiles of tr rows times chunk groups (0 when there is
// nothing to do).
static inline int64_t grid_x(const AttendArgs& a, int tr) {
  const int64_t tiles = ((int64_t)a.n_q * a.G + tr - 1) / tr;
  return tiles * a.ngroups;
}

static inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Prepared query rows in a workspace, after the partials: [rotated f32 query rows x D] [int8
// query rows x D] [scale f32 rows] [block sums int32 rows x D / 32], then room for the rotated f32
// K and V rows of a chunk (full-precision prefill, Hadamard layout: at most `rows` rows each, the
// chunk having n_q * Hkv <= rows of them), each part 16-byte aligned.
struct RowPrep {
  size_t qrot, q8, sq, qsum, kc, vc, end;
};

static inline RowPrep row_prep_layout(size_t at, size_t rows, int D) {
  RowPrep w;
  w.qrot = align16(at);
  w.q8 = w.qrot + align16(rows * D * sizeof(float));
  w.sq = w.q8 + align16(rows * D);
  w.qsum = w.sq + align16(rows * sizeof(float));
  w.kc = w.qsum + align16(rows * (D / 32) * sizeof(int));
  w.vc = w.kc + align16(rows * D * sizeof(float));
  w.end = w.vc + align16(rows * D * sizeof(float));
  return w;
}

// Query preparation of n_vec rows of q (kvq_prefill.hip): int8 query, scale, block sums, and for
// the Hadamard layout the rotated f32 query.  Points a's prepared-row fields at them.
kvq_status launch_prepare_rows(const kvq_cache* c, const float* q, int n_vec, unsigned char* ws, const RowPrep& w,
                               AttendArgs& a, hipStream_t s);

// Hadamard rotation of f32 K and V rows [n_tok][Hkv][D] without storing them (kvq_store.hip).
kvq_status launch_rotate_rows(const kvq_cache* c, const float* k_new, const float* v_new, int n_tok, float* kr,
                              float* vr, hipStream_t st);

// The online-softmax reduce over the partials of batch * rows_per_b rows (kvq_attend.hip);
// nwin_always > 0: the rows' f32-row partials are the last nwin_always slots (full-precision
// prefill, slices of `slice` rows; with causal_nq > 0, the causal limit of query i, i = (row in the
// batch row) / (rows_per_b / causal_nq), reaches only the first (W + i) / slice + 1 of them, W the
// row's window); else one window partial when n_recent > 0 and the row is not empty.  narrow: the
// records are the prefill's (narrow_stride), else the decode's f32 ones (partial_stride).
kvq_status launch_reduce(const kvq_cache* c, float* out, int32_t batch, int32_t rows_per_b, const int32_t* seq_len,
                         int nc1, int32_t chunk, const float* ws, hipStream_t s, int nwin_always = 0, int slice = 0,
                         int causal_nq = 0, RunSplit rs = RunSplit{}, bool narrow = false);

// The decode's two phases (kvq_attend.hip), for kvq_attend_decode and its variants: decode_check
// validates the arguments; decode_partial_ws and decode_reduce_ws then run the split-K phase and the
// merge with the partials in `workspace`, which must hold decode_partials_bytes(...) bytes.
kvq_status decode_check(const kvq_cache* c, const float* q, int32_t batch, int32_t Hq, const int32_t* block_table,
                        int32_t max_pages, const int32_t* seq_len, int32_t max_seq_len, int32_t chunk);
size_t decode_partials_bytes(const kvq_cache* c, int batch, int Hq, int max_seq_len, int chunk);
kvq_status decode_partial_ws(const kvq_cache* c, const float* q, int32_t batch, int32_t Hq, float alpha,
                             const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                             int32_t max_seq_len, int32_t chunk, void* workspace, void* stream, bool fq);
kvq_status decode_reduce_ws(const kvq_cache* c, float* out, int32_t batch, int32_t Hq, const int32_t* seq_len,
                            int32_t max_seq_len, int32_t chunk, const void* workspace, void* stream, bool fq = false);

}  // namespace kvq
