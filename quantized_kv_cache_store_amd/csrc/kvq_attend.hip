// Fused compressed-domain attention over the packed cache: the split-K partial
// kernel (decode and causal prefill), the f32 window partial, and the
// online-softmax reduce.
//
// [Open-TQ-Metal] Algorithm 1 (fused single pass over the packed cache, no
// dequantised S x d temporary) and the split-K paragraphs (chunks in parallel,
// each emitting o_c, m_c, l_c; a second phase merges them).  Scores are the
// integer dot int8(Q) . code(K) per 32-element block with the scales applied
// outside the reduction ([tract-RFC] Architecture > Data flow (decode)).
//
// Rows.  The kernels work on "rows": one query vector of one query head.  A
// batch entry with n_q queries has n_q * G rows per kv head (G = GQA group),
// row R = i * G + g for query i and head hk * G + g.  Decode is n_q = 1, so a kv
// head's rows are its G heads; causal prefill ([tract-RFC] Architecture,
// prefill) gives row R the limit q_start + i: it sees tokens t <= that limit.
// Sixteen consecutive rows form a tile, which is the N side of the MFMAs.
//
// gfx950 mapping.  One block of four waves handles one (batch row, kv head,
// row tile, four consecutive chunks); each wave takes 32-token steps of its
// chunk.  For a step:
//   * Q K^T runs on v_mfma_i32_16x16x32_i8: A = 16 tokens x 32 codes of one
//     block (unpacked nibbles, one dword per lane), B = the int8 query of the
//     tile's 16 rows (kept in registers for the block).  The i32 result per
//     (token, row, block) is scaled by the block's scale.
//   * P V runs on v_mfma_f32_16x16x32_f16 with the output transposed,
//     C[d][row] += V^T[d][t] P^T[t][row]: the P^T operand is exactly the
//     softmax numerators the lane already holds from Q K^T (lane = row,
//     k-slots = its 8 tokens), so no shuffle is needed; the V^T operand is
//     built from the packed dwords of the same 8 tokens, nibble p of dword c
//     giving row d = 8c + p (fp16 "1024 + code" then an exact offset and the
//     block scale).
//   * the online softmax keeps m and l per row in the lanes that own the
//     row's column, so the rescale of the accumulators is lane-local.
// Causal skip ([tract-RFC] Causality & mixed precision): a wave stops at the
// last token any row of its tile can see, and a chunk wholly past every
// limit streams nothing and emits the empty partial (m = -inf, l = 0, o = 0).
// Steps that are partly visible mask per row.  With the skip off, the masked
// tokens are streamed and contribute exact zeros, so both give the same bits.

#include "kvq_attend_common.h"

namespace kvq {

// Staging buffer of one 32-token step in a wave's LDS slice:
//   [K payload rows 32 x RS][V payload rows 32 x RS][K records 32 x SB][V records 32 x SB]
// with payload rows padded to RS = PB + 16 bytes, which spreads the reads of a 16-row column
// (K: one dword per lane from 16 rows; V: 16 dwords of one row times four rows 4 apart) over
// all 64 LDS banks.
// filled from registers that were loaded one step ahead with 16-byte loads.
template <int L, int D>
struct Step {
  using T = Layout<L, D>;
  static constexpr int PB = T::PB, SB = T::SB;
  static constexpr int RS = PB + 16;
  static constexpr int KP = 0, VP = 32 * RS, KR = 64 * RS, VR = KR + 32 * SB;
  static constexpr int BYTES = VR + 32 * SB;
  static constexpr int PAY_SLOTS = (2 * PB + 63) / 64;   // 16-byte chunks of 32 payload rows, per lane
  static constexpr int REC_SLOTS = (4 * SB + 63) / 64;   // K and V records together
  static constexpr int SLOTS = 2 * PAY_SLOTS + REC_SLOTS;
};

// Physical row indices of the two 16-token halves of the step at T (wave-uniform).
struct HalfRows {
  size_t r0, r1;
};

// Page entries of a wave's chunk held in registers (entry i in lane i % 64 of register i / 64), so
// that a step's rows come from readlane on the scalar unit: the streaming loop then issues no
// memory operation other than its own 16-byte loads, which keeps the load-counter waits exact.
constexpr int kPageRegs = 4;   // up to 256 pages per chunk

struct ChunkPages {
  int first_page;
  int lane_page[kPageRegs];
};

__device__ __forceinline__ ChunkPages chunk_pages(const AttendArgs& a, int b, int t_begin, int t_end, int lane,
                                                  bool active) {
  ChunkPages cp;
  cp.first_page = t_begin >> a.page_shift;
  const int npages = active ? ((t_end - 1) >> a.page_shift) - cp.first_page + 1 : 0;
#pragma unroll
  for (int i = 0; i < kPageRegs; ++i) {
    const int e = lane + 64 * i;
    cp.lane_page[i] = e < npages ? a.block_table[(size_t)b * a.max_pages + cp.first_page + e] : 0;
  }
  return cp;
}

__device__ __forceinline__ size_t chunk_row(const AttendArgs& a, const ChunkPages& cp, int hk, int t) {
  const int e = (t >> a.page_shift) - cp.first_page;     // wave-uniform
  int phys = __builtin_amdgcn_readlane(cp.lane_page[0], e & 63);
#pragma unroll
  for (int i = 1; i < kPageRegs; ++i)
    if ((e >> 6) == i) phys = __builtin_amdgcn_readlane(cp.lane_page[i], e & 63);
  return (((size_t)phys * a.Hkv + hk) << a.page_shift) + (size_t)(t & ((1 << a.page_shift) - 1));
}

__device__ __forceinline__ HalfRows half_rows(const AttendArgs& a, const ChunkPages& cp, int hk, int T, int t_end,
                                              size_t row_first) {
  HalfRows h;
  h.r0 = T < t_end ? chunk_row(a, cp, hk, T) : row_first;
  h.r1 = T + 16 < t_end ? chunk_row(a, cp, hk, T + 16) : row_first;
  return h;
}

// Issue the 16-byte loads of one step into pre[] (no wait).  Payload chunk ci of the step is
// row ci / PB (half ci / PB), bytes 16 * (ci % PB); when PB is a multiple of 64 every slot lies in
// one half, so its base address is wave-uniform and only lane * 16 varies.
// The cache is read once per decode step, so every load carries the nontemporal hint (measured on
// this access pattern: 5.7 -> 6.2 TB/s on loads alone).
__device__ __forceinline__ u32x4 stream_load(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int L, int D>
__device__ __forceinline__ void issue_step(const AttendArgs& a, HalfRows hr, int lane, u32x4* pre, bool dummy = false) {
  using ST = Step<L, D>;
  constexpr int PB = ST::PB, SB = ST::SB;
  if (dummy) lane = 0;
#pragma unroll
  for (int k = 0; k < ST::PAY_SLOTS; ++k) {
    if (PB % 64 == 0 || dummy) {
      const int half = (64 * k) / PB;                     // compile-time
      const size_t row = half ? hr.r1 : hr.r0;
      const size_t off = dummy ? hr.r0 * PB : row * PB + (size_t)((64 * k) % PB) * 16 + (size_t)lane * 16;
      pre[k] = stream_load(a.kp + off);
      pre[ST::PAY_SLOTS + k] = stream_load(a.vp + off);
    } else {
      const int ci = lane + 64 * k;
      if (ci < 2 * PB) {
        const size_t row = (ci >= PB) ? hr.r1 : hr.r0;
        const size_t off = row * PB + (size_t)(ci % PB) * 16;
        pre[k] = stream_load(a.kp + off);
        pre[ST::PAY_SLOTS + k] = stream_load(a.vp + off);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < ST::REC_SLOTS; ++k) {
    const int ci = dummy ? 0 : lane + 64 * k;
    if (ci < 4 * SB) {
      const int cc = ci % (2 * SB);                 // chunk within the tensor's 32 records
      const size_t row = (cc >= SB) ? hr.r1 : hr.r0;
      const uint8_t* base = ci < 2 * SB ? a.ks : a.vs;
      pre[2 * ST::PAY_SLOTS + k] = stream_load(base + row * SB + (size_t)(cc % SB) * 16);
    }
  }
}

template <int L, int D>
__device__ __forceinline__ void stage_step(unsigned char* buf, int lane, const u32x4* pre) {
  using ST = Step<L, D>;
  constexpr int PB = ST::PB, SB = ST::SB;
#pragma unroll
  for (int k = 0; k < ST::PAY_SLOTS; ++k) {
    const int ci = lane + 64 * k;
    if (ci < 2 * PB) {
      const int at = (ci / (PB / 16)) * ST::RS + (ci % (PB / 16)) * 16;   // row ci / (PB / 16), padded
      *reinterpret_cast<u32x4*>(buf + ST::KP + at) = pre[k];
      *reinterpret_cast<u32x4*>(buf + ST::VP + at) = pre[ST::PAY_SLOTS + k];
    }
  }
#pragma unroll
  for (int k = 0; k < ST::REC_SLOTS; ++k) {
    const int ci = lane + 64 * k;
    if (ci < 4 * SB) *reinterpret_cast<u32x4*>(buf + ST::KR + ci * 16) = pre[2 * ST::PAY_SLOTS + k];
  }
}

// f16 element idx of a record, as f32
__device__ __forceinline__ float rec_f16(const unsigned char* p, int idx) {
  return (float)reinterpret_cast<const _Float16*>(p)[idx];
}

// Record word idx of a staged record as f16 pairs (scale, or scale|zero for asym).
__device__ __forceinline__ uint32_t rec_word(const unsigned char* rec, int idx) {
  return reinterpret_cast<const uint32_t*>(rec)[idx];
}

// One 32-token step of a wave: Q K^T, online softmax, P V, all from the staged rows in `buf`.
// FULL: every token of the step is inside the chunk and visible to every row (no masking).
// Otherwise tokens at or past t_end are dropped (their staged rows may hold anything, so their
// scales are zeroed too) and tokens past `lim`, the limit of this lane's row, get p = 0.
// drow: flat row index of this lane's row for the score export (DBG), or -1.
template <int L, int D, bool DBG, bool FULL>
__device__ __forceinline__ void attend_step(const AttendArgs& a, const unsigned char* buf, int T0, int t_end,
                                            int lim, long drow, int col, int r, const long* qB,
                                            const float* qsB, const int* qoff, float sqc, uint32_t magic,
                                            float& m_run, float& l_run, v4f* oacc) {
  using T = Layout<L, D>;
  using ST = Step<L, D>;
  constexpr int NG = T::NG;
  constexpr int SG = T::SG;
  constexpr int PB = T::PB, SB = T::SB;
  constexpr int NO = D / 128;
  constexpr int BIAS = CodeBias<L>::value;

  // ---------------- Q K^T on the int8 MFMA, scores of this lane's 8 tokens
  float xs[8];
  float vs_had[8];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const unsigned char* krow = buf + ST::KP + (16 * tau + col) * ST::RS;
    v4i acc[SG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      uint32_t lo, hi;
      if (L == Q60) {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(krow + 24 * g + 4 * r);
        const uint32_t t2 = *reinterpret_cast<const uint16_t*>(krow + 24 * g + 16 + 2 * r);
        q6_octet(x, t2, lo, hi);
      } else {
        uint32_t x = *reinterpret_cast<const uint32_t*>(krow + 4 * (4 * g + r));
        if (BIAS) x ^= 0x88888888u;
        lo = x & 0x0F0F0F0Fu;
        hi = (x >> 4) & 0x0F0F0F0Fu;
      }
      const long A = __builtin_bit_cast(long, u32x2{lo, hi});
      const long B = qB[g];
      if (L == HAD) {
        acc[0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, g == 0 ? v4i{0, 0, 0, 0} : acc[0], 0, 0, 0);
      } else {
        acc[g] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, v4i{0, 0, 0, 0}, 0, 0, 0);
      }
    }
    // offset term: A[t = col][k = r] from the record of token 16*tau + col
    v4f xo = v4f{0.f, 0.f, 0.f, 0.f};
    if (L != HAD) {
      const unsigned char* orec = buf + ST::KR + (16 * tau + col) * SB;
#pragma unroll
      for (int i = 0; i < NG / 4; ++i) {
        const float av = (L == ASYM) ? rec_f16(orec, 2 * (4 * i + r) + 1) : rec_f16(orec, 4 * i + r);
        xo = __builtin_amdgcn_mfma_f32_16x16x4f32(av, qsB[i], xo, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = 16 * tau + 4 * r + j;       // token within the step
      const bool ok = FULL || T0 + tl < t_end;
      const bool vis = FULL || (ok && T0 + tl <= lim);
      const unsigned char* rec = buf + ST::KR + tl * SB;
      float x;
      if (L == HAD) {
        const int I = acc[0][j] - qoff[0];
        x = *reinterpret_cast<const float*>(rec) * (float)I;
        if (DBG && ok && drow >= 0) a.dbg[(size_t)drow * a.max_seq_len + T0 + tl] = I;
        const float vsc = *reinterpret_cast<const float*>(buf + ST::VR + tl * SB);
        vs_had[tau * 4 + j] = ok ? vsc : 0.0f;
      } else {
        x = xo[j];
#pragma unroll
        for (int g = 0; g < SG; ++g) {
          // scale of block g: low half of word g (asym: scale|zero), or half g of the packed fp16 scales
          const uint32_t w = rec_word(rec, (L == ASYM) ? g : (g >> 1));
          const float s = (float)as_h2(w)[(L == ASYM) ? 0 : (g & 1)];
          x = fmaf(s, (float)acc[g][j], x);
          if (DBG && ok && drow >= 0)
            a.dbg[((size_t)drow * a.max_seq_len + T0 + tl) * SG + g] = acc[g][j] - qoff[g];
        }
      }
      xs[tau * 4 + j] = vis ? x * sqc : -INFINITY;
    }
  }
  if (DBG) return;

  // ---------------- online softmax (base 2), per head = lane column
  float smax = xs[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) smax = fmaxf(smax, xs[i]);
  smax = max_over_rows(smax);
  const float m_new = fmaxf(m_run, smax);
  const float m_use = m_new == -INFINITY ? 0.0f : m_new;
  // rescale the running sums only when some lane's maximum moved (rare after the first steps)
  if (__any(m_new > m_run)) {
    const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
    l_run *= corr;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[i] *= corr;
  }
  m_run = m_new;
  float psum = 0.0f;
  v8h pB;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = __builtin_amdgcn_exp2f(xs[i] - m_use);
    psum += p;
    pB[i] = (_Float16)(L == HAD ? p * vs_had[i] : p);
  }
  l_run += psum;

  // ---------------- P V on the f16 MFMA, V^T built from the staged rows
#pragma unroll
  for (int o = 0; o < NO; ++o) {
    const int oc = col + 16 * o;       // this lane's octet (elements 8*oc .. 8*oc+7)
    const int grp = oc >> 2;           // its 32-element block
    uint32_t ev[8], od[8];
    uint32_t sz[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int tl = 16 * (k >> 2) + 4 * r + (k & 3);
      const unsigned char* vrow = buf + ST::VP + tl * ST::RS;
      if (L == Q60) {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(vrow + 24 * grp + 4 * (oc & 3));
        const uint32_t t2 = *reinterpret_cast<const uint16_t*>(vrow + 24 * grp + 16 + 2 * (oc & 3));
        q6_octet(x, t2, ev[k], od[k]);
      } else {
        uint32_t x = *reinterpret_cast<const uint32_t*>(vrow + 4 * oc);
        if (BIAS) x ^= 0x88888888u;
        ev[k] = x;
        od[k] = 0;
      }
      const bool ok = FULL || T0 + tl < t_end;   // rows past the end may hold anything: zero their scale
      const unsigned char* vrec = buf + ST::VR + tl * SB;
      uint32_t v;
      if (L == ASYM) v = reinterpret_cast<const uint32_t*>(vrec)[grp];
      else if (L != HAD) v = (uint32_t)reinterpret_cast<const uint16_t*>(vrec)[grp];
      else v = 0u;
      sz[k] = ok ? v : 0u;
    }
    h2 s2[4], z2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s2[i] = as_h2(__builtin_amdgcn_perm(sz[2 * i + 1], sz[2 * i], 0x05040100u));
      z2[i] = as_h2(__builtin_amdgcn_perm(sz[2 * i + 1], sz[2 * i], 0x07060302u));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v8h A;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t bsel = (uint32_t)(e >> 1);
        const uint32_t sel = bsel | (0x0Cu << 8) | ((4u + bsel) << 16) | (0x0Cu << 24);
        uint32_t pair;
        if (L == Q60) {
          const uint32_t src_a = (e & 1) ? od[2 * i] : ev[2 * i];
          const uint32_t src_b = (e & 1) ? od[2 * i + 1] : ev[2 * i + 1];
          pair = __builtin_amdgcn_perm(src_b, src_a, sel) | magic;
        } else {
          const uint32_t y = __builtin_amdgcn_perm(ev[2 * i + 1], ev[2 * i], sel);
          pair = (((e & 1) ? (y >> 4) : y) & 0x000F000Fu) | magic;
        }
        h2 v = as_h2(pair) - h2{(_Float16)(1024 + BIAS), (_Float16)(1024 + BIAS)};
        if (L == ASYM) v = v * s2[i] + z2[i];
        else if (L != HAD) v = v * s2[i];
        A[2 * i] = v[0];
        A[2 * i + 1] = v[1];
      }
      oacc[o * 8 + e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pB, oacc[o * 8 + e], 0, 0, 0);
    }
  }
}

// Split-K partial kernel.  Block = four waves = four consecutive chunks of one (batch row,
// kv head, row tile); each wave streams its chunk in 32-token steps with NB - 1 steps of loads
// in flight and writes the chunk's partial per row (o unnormalised, m in base-2 logits, l).
// Grid: x = row tile * ngroups + chunk group (the last group is the window when n_recent > 0),
// y = kv head, z = batch row.
template <int L, int D, bool DBG>
__global__ __launch_bounds__(256, 2) void attend_partial(AttendArgs a) {
  using T = Layout<L, D>;
  using ST = Step<L, D>;
  constexpr int NB = (ST::SLOTS <= 5) ? 5 : (D == 128 ? 3 : 2);   // ring slots: NB - 1 steps in flight while one is consumed
  constexpr int NG = T::NG;
  constexpr int SG = T::SG;
  constexpr int NO = D / 128;
  constexpr int BIAS = CodeBias<L>::value;
  extern __shared__ __align__(16) unsigned char smem[];

  // Block numbering: chunk group fastest (measured faster than kv head or batch row fastest: blocks
  // that run together then stream neighbouring chunks of one (row, kv head)).
  const int hk = blockIdx.y, b = blockIdx.z;
  const int tile = (int)blockIdx.x / a.ngroups;
  const int cg = (int)blockIdx.x - tile * a.ngroups;
  const int S = a.seq_len[b];
  const int Sq = a.n_recent > 0 ? max(0, S - a.n_recent) : S;   // quantised tokens
  const int nrows = a.n_q * a.G;
  const int row0 = 16 * tile;
  const int nvalid = min(16, nrows - row0);
  const int qs0 = a.causal ? a.q_start[b] : 0;
  if (!DBG && a.n_recent > 0 && cg == a.ngroups - 1) {
    if (S > 0) window_partial<L, D>(a, smem, b, hk, S, row0, nvalid, qs0);
    return;
  }
  if (cg * 4 * a.chunk >= Sq) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = cg * 4 + wave;                  // this wave's chunk
  const int t_begin = c * a.chunk;
  const int lim_min = row_limit(a, qs0, row0, nrows);               // first row of the tile
  const int lim_max = row_limit(a, qs0, row0 + nvalid - 1, nrows);  // last row: the tile's farthest limit
  int t_end = min(t_begin + a.chunk, Sq);
  if (a.skip && lim_max < t_end - 1) t_end = max(t_begin, lim_max + 1);   // causal skip
  const bool has_chunk = t_begin < Sq;          // the reduce reads this chunk's partial (wave-uniform)
  const bool active = t_begin < t_end;          // tokens to stream
  const ChunkPages cp = chunk_pages(a, b, t_begin, t_end, lane, active);
  const size_t row_first = active ? chunk_row(a, cp, hk, t_begin) : 0;
  const int nsteps = active ? (t_end - t_begin + 31) / 32 : 0;

  u32x4 pre[NB][ST::SLOTS];

  // ---- prologue: this lane's row of the tile from the prepared rows (int8 query in the B-operand
  // order, its scale and block sums); the perms and sums consume the loads here, before the loop
  const int col = lane & 15;
  const int r = lane >> 4;
  long qB[NG];   // B operands (int8 query of the tile's rows), one aligned register pair each
  float qsB[NG / 4];   // offset-term operand: zero point (asym) or -bias * scale times the block sums
  int qoff[SG];        // bias * sum(q8): the Hadamard scores and the score export use it
  float sqc = 0.0f;
  {
    const size_t fr = row_index(a, b, hk, row0 + min(col, nvalid - 1));
    const int* qs = a.qsump + fr * NG;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint2 w = *reinterpret_cast<const uint2*>(a.q8p + fr * D + 32 * g + 8 * r);
      qB[g] = __builtin_bit_cast(long, u32x2{__builtin_amdgcn_perm(w.y, w.x, 0x06040200u),
                                             __builtin_amdgcn_perm(w.y, w.x, 0x07050301u)});
    }
#pragma unroll
    for (int i = 0; i < NG / 4; ++i) qsB[i] = (L == ASYM) ? (float)qs[4 * i + r] : -(float)BIAS * (float)qs[4 * i + r];
#pragma unroll
    for (int g = 0; g < SG; ++g) {
      int sum = 0;
      if (L == HAD) {
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) sum += qs[gg];
      } else {
        sum = qs[g];
      }
      qoff[g] = BIAS * sum;
    }
    sqc = a.sqp[fr] * a.alpha * KVQ_LOG2E;
  }
  const int lim = row_limit(a, qs0, row0 + col, nrows);
  const long drow = (DBG && col < nvalid) ? (long)row_index(a, b, hk, row0 + col) : -1;   // score export only
  if (!has_chunk) return;

  unsigned char* buf = smem + wave * ST::BYTES;
  float m_run = -INFINITY, l_run = 0.0f;
  v4f oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  uint32_t magic;   // fp16 "1024 + code" exponent bits, kept in a VGPR so v_and_or_b32 can take it
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
  // Software pipeline over a ring of NB register slots, all loads issued inside the loop (nothing is
  // in flight at entry, so the compiler's load-counter waits stay exact): iteration i issues step i
  // into slot i % NB and consumes step i - (NB - 1) from slot (i + 1) % NB.  Issues past the last
  // step read a few bytes of the chunk's first rows (cache hits) so every iteration issues the same
  // loads.
  const int kend = nsteps > 0 ? nsteps + NB - 1 : 0;
  for (int k0 = 0; k0 < kend; k0 += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int si = k0 + k;
      const int Ti = t_begin + 32 * si;
      issue_step<L, D>(a, half_rows(a, cp, hk, Ti, t_end, row_first), lane, pre[k], si >= nsteps);
      const int su = si - (NB - 1);
      if (su >= 0 && su < nsteps) {
        const int T = t_begin + 32 * su;
        stage_step<L, D>(buf, lane, pre[(k + 1) % NB]);
        if (T + 32 <= t_end && T + 31 <= lim_min)
          attend_step<L, D, DBG, true>(a, buf, T, t_end, lim, drow, col, r, qB, qsB, qoff, sqc, magic, m_run, l_run, oacc);
        else
          attend_step<L, D, DBG, false>(a, buf, T, t_end, lim, drow, col, r, qB, qsB, qoff, sqc, magic, m_run, l_run, oacc);
      }
    }
  }
  if (DBG) return;

  // ---------------- this wave's chunk partial
  l_run = sum_over_rows(l_run);
  if (col < nvalid) {
    float* dst = a.ws + (row_index(a, b, hk, row0 + col) * a.nc1 + c) * partial_stride(D);
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[8 * (4 * r + j + 16 * o) + e] = oacc[o * 8 + e][j];
    if (r == 0) {
      dst[D] = m_run;
      dst[D + 1] = l_run;
    }
  }
}

// Online-softmax merge of the chunk partials of each row (flat index (b * n_q + i) * Hq + h);
// Hadamard layout: rotate back.  W waves per row (4 / W rows per block): the row's waves split
// its chunks and, when W > 1, combine through LDS in a fixed order (deterministic).  Lane l owns
// output elements l * E .. l * E + E - 1; the rotation runs in registers, butterflies inside a
// lane for strides below E and between lanes above, in the stage order of the encoding
// (h = 1, 2, ..., D / 2, then 1 / sqrt(D)).
template <int D, bool ROT, int W>
__global__ __launch_bounds__(256) void attend_reduce(const float* ws, float* out, const int32_t* seq_len,
                                                     int rows_per_b, int nc1, int chunk, int n_recent,
                                                     long total_rows) {
#pragma clang fp contract(off)
  constexpr int E = D / 64;
  constexpr int RPB = 4 / W;
  __shared__ float red_o[4][D];
  __shared__ float red_m[4], red_l[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = wave % W;
  const long row = (long)blockIdx.x * RPB + wave / W;
  const bool valid = row < total_rows;              // wave-uniform
  const long rr = valid ? row : total_rows - 1;
  const int b = (int)(rr / rows_per_b);
  const int S = seq_len[b];
  const int Sq = n_recent > 0 ? max(0, S - n_recent) : S;
  const int nq = (Sq + chunk - 1) / chunk;
  const int cnt = nq + ((n_recent > 0 && S > 0) ? 1 : 0);
  const int PST = partial_stride(D);
  const float* base = ws + (size_t)rr * nc1 * PST;
  float M = -INFINITY;
  for (int i = sub * 64 + lane; i < cnt; i += 64 * W) M = fmaxf(M, base[(size_t)(i < nq ? i : nc1 - 1) * PST + D]);
  for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m));
  if (W > 1) {
    if (lane == 0) red_m[wave] = M;
    __syncthreads();
    const int w0 = wave - sub;
    M = red_m[w0];
    for (int k = 1; k < W; ++k) M = fmaxf(M, red_m[w0 + k]);
  }
  float o[E], l = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.0f;
#pragma unroll 4
  for (int i = sub; i < cnt; i += W) {
    const float* p = base + (size_t)(i < nq ? i : nc1 - 1) * PST;
    const float mc = p[D];
    const float w = (mc == -INFINITY) ? 0.0f : exp2f(mc - M);
    l += w * p[D + 1];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] += w * p[lane * E + e];
  }
  if (W > 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) red_o[wave][lane * E + e] = o[e];
    if (lane == 0) red_l[wave] = l;
    __syncthreads();
    if (sub != 0) return;
    l = red_l[wave];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = red_o[wave][lane * E + e];
    for (int k = 1; k < W; ++k) {
      l += red_l[wave + k];
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += red_o[wave + k][lane * E + e];
    }
  }
  if (!valid) return;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = l > 0.0f ? o[e] / l : 0.0f;
  if (ROT) {
#pragma unroll
    for (int h = 1; h < E; h <<= 1) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if ((e & h) == 0) {
          const float a = x[e], c = x[e + h];
          x[e] = a + c;
          x[e + h] = a - c;
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {   // stride m * E: partner lane differs in bit m
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float y = __shfl_xor(x[e], m);
        x[e] = upper ? (y - x[e]) : (x[e] + y);
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = x[e] * hadamard_norm<D>();
  }
#pragma unroll
  for (int e = 0; e < E; ++e) out[(size_t)row * D + lane * E + e] = x[e];
}

template <int L, int D, bool DBG>
static void launch_partial(const AttendArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  if (lds > 65536)
    (void)hipFuncSetAttribute((const void*)attend_partial<L, D, DBG>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((attend_partial<L, D, DBG>), grid, dim3(256), lds, st, a);
}

typedef void (*partial_fn)(const AttendArgs&, dim3, size_t, hipStream_t);

template <bool DBG>
static partial_fn pick_partial(int layout, int D) {
  const int di = D == 256 ? 1 : 0;
  static const partial_fn tab[4][2] = {
      {launch_partial<HAD, 128, DBG>, launch_partial<HAD, 256, DBG>},
      {launch_partial<Q40, 128, DBG>, launch_partial<Q40, 256, DBG>},
      {launch_partial<Q60, 128, DBG>, launch_partial<Q60, 256, DBG>},
      {launch_partial<ASYM, 128, DBG>, launch_partial<ASYM, 256, DBG>},
  };
  return tab[layout][di];
}

static size_t step_bytes(int layout, int D) {
  return 64 * (payload_bytes_rt(layout, D) + 16 + scale_bytes_rt(layout, D));
}

static size_t partial_lds_bytes(int layout, int D, int n_recent) {
  const size_t steps = 4 * step_bytes(layout, D);
  const size_t win = n_recent > 0 ? (size_t)(D == 128 ? window_lds_bytes<128>() : window_lds_bytes<256>()) : 0;
  return steps > win ? steps : win;
}

// Workspace of the decode: the partials [B x Hq x (chunks + 1) x (D + 4)] f32, then the prepared rows.
static RowPrep decode_ws(int batch, int Hq, int D, int max_seq_len, int chunk) {
  const size_t rows = (size_t)batch * Hq;
  const size_t nc1 = (size_t)chunks_of(max_seq_len, chunk) + 1;
  return row_prep_layout(rows * nc1 * partial_stride(D) * sizeof(float), rows, D);
}

static kvq_status check_chunk(const kvq_cache* c, int32_t chunk) {
  if (chunk < 128 || chunk % 128) return fail(KVQ_ERR_INVALID_ARG, "chunk_tokens must be a positive multiple of 128");
  if ((chunk + c->page_size - 1) / c->page_size + 1 > 64 * kPageRegs)
    return fail(KVQ_ERR_UNSUPPORTED, "a chunk may span at most %d pages", 64 * kPageRegs - 1);
  return KVQ_OK;
}

template <int D, bool ROT, int W>
static void launch_reduce_w(float* out, long rows, int rows_per_b, const int32_t* seq_len, int nc1, int chunk,
                            int n_recent, const float* ws, hipStream_t s) {
  const long blocks = (rows + (4 / W) - 1) / (4 / W);
  hipLaunchKernelGGL((attend_reduce<D, ROT, W>), dim3((unsigned)blocks), dim3(256), 0, s, ws, out, seq_len, rows_per_b,
                     nc1, chunk, n_recent, rows);
}

kvq_status launch_reduce(const kvq_cache* c, float* out, int32_t batch, int32_t rows_per_b, const int32_t* seq_len,
                         int nc1, int32_t chunk, const float* ws, hipStream_t s) {
  const long rows = (long)batch * rows_per_b;
  // one wave per row when there are rows enough to fill the chip, else four waves split each row
  const bool many = rows >= 4096;
  const bool rot = c->layout == HAD;
  const int n = c->n_recent;
  if (c->head_dim == 128) {
    if (rot) many ? launch_reduce_w<128, true, 1>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s)
                  : launch_reduce_w<128, true, 4>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s);
    else many ? launch_reduce_w<128, false, 1>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s)
              : launch_reduce_w<128, false, 4>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s);
  } else {
    if (rot) many ? launch_reduce_w<256, true, 1>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s)
                  : launch_reduce_w<256, true, 4>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s);
    else many ? launch_reduce_w<256, false, 1>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s)
              : launch_reduce_w<256, false, 4>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s);
  }
  return check_launch("attention reduce kernel");
}

}  // namespace kvq

using namespace kvq;

extern "C" size_t kvq_decode_workspace_bytes(int32_t batch, int32_t Hq, int32_t D, int32_t max_seq_len,
                                             int32_t chunk) {
  if (batch < 1 || Hq < 1 || (D != 128 && D != 256) || max_seq_len < 0 || chunk < 128 || chunk % 128) return 0;
  // +1 partial slot for the window (always reserved so the size does not depend on n_recent)
  return decode_ws(batch, Hq, D, max_seq_len, chunk).end;
}

extern "C" kvq_status kvq_attend_decode_partial(const kvq_cache* c, const float* q, int32_t batch, int32_t Hq,
                                                float alpha, const int32_t* block_table, int32_t max_pages,
                                                const int32_t* seq_len, int32_t max_seq_len, int32_t chunk,
                                                void* workspace, size_t ws_bytes, void* stream) {
  kvq_status st = check_attend_args(c, q, batch, Hq, block_table, max_pages, seq_len, max_seq_len);
  if (st != KVQ_OK) return st;
  if ((st = check_chunk(c, chunk)) != KVQ_OK) return st;
  const size_t need = kvq_decode_workspace_bytes(batch, Hq, c->head_dim, max_seq_len, chunk);
  if (!workspace || ws_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  AttendArgs a = make_args(c, q, Hq, 1, alpha, block_table, max_pages, seq_len, max_seq_len, chunk, workspace);
  const int64_t gx = grid_x(a);
  if (gx == 0) return KVQ_OK;
  if ((st = launch_prepare_rows(c, q, batch * Hq, (unsigned char*)workspace,
                                decode_ws(batch, Hq, c->head_dim, max_seq_len, chunk), a, (hipStream_t)stream)) != KVQ_OK)
    return st;
  a.batch = batch;
  const dim3 grid((unsigned)gx, c->num_kv_heads, batch);
  pick_partial<false>(c->layout, c->head_dim)(a, grid, partial_lds_bytes(c->layout, c->head_dim, c->n_recent), (hipStream_t)stream);
  return check_launch("decode partial kernel");
}

extern "C" kvq_status kvq_attend_decode_reduce(const kvq_cache* c, float* out, int32_t batch, int32_t Hq,
                                               const int32_t* seq_len, int32_t max_seq_len, int32_t chunk,
                                               const void* workspace, size_t ws_bytes, void* stream) {
  kvq_status st = validate_cache(c);
  if (st != KVQ_OK) return st;
  if (!out || !seq_len) return fail(KVQ_ERR_INVALID_ARG, "out and seq_len must be non-null");
  if (batch < 1 || Hq < 1 || Hq % c->num_kv_heads) return fail(KVQ_ERR_INVALID_ARG, "bad batch or num_q_heads");
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (chunk < 128 || chunk % 128) return fail(KVQ_ERR_INVALID_ARG, "chunk_tokens must be a positive multiple of 128");
  const size_t need = kvq_decode_workspace_bytes(batch, Hq, c->head_dim, max_seq_len, chunk);
  if (!workspace || ws_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  return launch_reduce(c, out, batch, Hq, seq_len, chunks_of(max_seq_len, chunk) + 1, chunk, (const float*)workspace,
                       (hipStream_t)stream);
}

extern "C" kvq_status kvq_attend_decode(const kvq_cache* c, const float* q, float* out, int32_t batch, int32_t Hq,
                                        float alpha, const int32_t* block_table, int32_t max_pages,
                                        const int32_t* seq_len, int32_t max_seq_len, int32_t chunk,
                                        void* workspace, size_t ws_bytes, void* stream) {
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out must be non-null");
  kvq_status st = kvq_attend_decode_partial(c, q, batch, Hq, alpha, block_table, max_pages, seq_len, max_seq_len,
                                            chunk, workspace, ws_bytes, stream);
  if (st != KVQ_OK) return st;
  return kvq_attend_decode_reduce(c, out, batch, Hq, seq_len, max_seq_len, chunk, workspace, ws_bytes, stream);
}

extern "C" kvq_status kvq_debug_qk_i32(const kvq_cache* c, const float* q, int32_t batch, int32_t Hq,
                                       const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                                       int32_t max_seq_len, int32_t* scores, void* workspace, size_t ws_bytes,
                                       void* stream) {
  kvq_status st = check_attend_args(c, q, batch, Hq, block_table, max_pages, seq_len, max_seq_len);
  if (st != KVQ_OK) return st;
  if (!scores) return fail(KVQ_ERR_INVALID_ARG, "scores must be non-null");
  const int chunk = 512;
  if ((st = check_chunk(c, chunk)) != KVQ_OK) return st;
  if (chunks_of(max_seq_len, chunk) == 0) return KVQ_OK;
  const size_t need = kvq_decode_workspace_bytes(batch, Hq, c->head_dim, max_seq_len, chunk);
  if (!workspace || ws_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  AttendArgs a = make_args(c, q, Hq, 1, 1.0f, block_table, max_pages, seq_len, max_seq_len, chunk, workspace);
  if ((st = launch_prepare_rows(c, q, batch * Hq, (unsigned char*)workspace,
                                decode_ws(batch, Hq, c->head_dim, max_seq_len, chunk), a, (hipStream_t)stream)) != KVQ_OK)
    return st;
  a.dbg = scores;
  a.kring = nullptr;
  a.vring = nullptr;
  a.ngroups = (chunks_of(max_seq_len, chunk) + 3) / 4;   // no window group: the export covers quantised tokens
  a.batch = batch;
  const dim3 grid((unsigned)grid_x(a), c->num_kv_heads, batch);
  pick_partial<true>(c->layout, c->head_dim)(a, grid, partial_lds_bytes(c->layout, c->head_dim, 0), (hipStream_t)stream);
  return check_launch("score export kernel");
}
