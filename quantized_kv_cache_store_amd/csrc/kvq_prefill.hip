// Causal prefill over the packed cache.
//
// [tract-RFC] Architecture (the prefill path stores the chunk first; attention
// then bounds each query by its own position) and Causality & mixed precision
// (skipping the work past a query's bound changes no bit of the result).  The scores are the same int8(Q) . code(K) -> i32 block
// dots as decode, and the window and merge are those of decode.
//
// Rows and tiles as in the decode kernel: row R of (batch b, kv head hk) is query
// i = R / G of head hk * G + R % G, with limit q_start + i.  A block of four
// waves takes 64 consecutive rows (one 16-row tile per wave) and one 1024-token
// chunk of the quantised region.  Unlike decode, where every wave streams its
// own chunk, here the block shares each 32-token step:
//   * the block unpacks the step's K codes once into LDS, already in the A-operand
//     order of v_mfma_i32_16x16x32_i8 (so a wave's operand is one contiguous
//     8-byte read per lane), and dequantises the step's V once into LDS as fp16,
//     already transposed into the A-operand order of v_mfma_f32_16x16x32_f16
//     (one contiguous 16-byte read per lane);
//   * each wave then runs Q K^T, the online softmax and P V for its tile from
//     those operands, so the unpack and dequantisation cost is paid once per
//     64 rows instead of once per 16.
// The step's global loads are issued one step ahead into registers; one barrier
// per step separates the producer writes of step s + 1 from the reads of step s
// (two LDS buffers).
//
// Causal skip: the block stops at the last token its last row can see, and a
// chunk wholly past every limit streams nothing and emits empty partials.  Steps
// that are partly visible mask per row.  With the skip off the masked tokens are
// streamed and contribute exact zeros, so both settings give the same bits.

#include <algorithm>
#include <map>
#include <type_traits>

#include "kvq_attend_common.h"

namespace kvq {

// Shortest split-K chunk of the prefill (tokens); each (row block, chunk) is one block of the grid.
constexpr int kPrefillChunk = 512;
// Full-precision prefill: its f32 rows (the prefix's window and the chunk's own rows) are split into
// slices of at least this many tokens, one group and one partial slot each.
constexpr int kRowSlice = 128;

// Slices of the f32 rows of a full-precision prefill of n_q queries (window at most n_recent).
static inline int row_slices(int n_recent, int n_q) { return (n_recent + n_q + kRowSlice - 1) / kRowSlice; }
static_assert(kPrefillChunk % 32 == 0, "chunks of whole 32-token steps");

// LDS of one 32-token step:
//   KC  int8 codes (code + bias; the Hadamard layout signed) in A-operand order: [block g][half tau][lane group r][token
//       16 tau + i][8 bytes], the bytes being codes 8r, 8r+2, 8r+4, 8r+6, 8r+1, 8r+3, 8r+5, 8r+7
//       of block g (8-bit layout: the signed codes 8r .. 8r+7 in order);
//   VT  dequantised V (fp16) in A-operand order of V^T: [d / 16][lane group r][d % 16][slot k],
//       slot k holding token 16 (k / 4) + 4r + k % 4 (the same token order as the lane's P);
//   KR  the raw K records of the 32 tokens;
//   VR  Hadamard layout: the f32 V scales of the 32 tokens (zero past the chunk's end), which its
//       consumers fold into P (VT then holds the bare codes).
template <int L, int D>
struct PStep {
  using T = Layout<L, D>;
  static constexpr int KC = 0;
  static constexpr int VT = KC + T::NG * 1024;
  static constexpr int KR = VT + D * 64;
  static constexpr int VR = KR + 32 * T::SB;
  static constexpr int BYTES = VR + (L == HAD ? 32 * 4 : 0);
  static constexpr int KU = T::NG / 2;        // K units (token, block, lane group) per thread
  static constexpr int VU = D / 128;          // V units (element pair, lane group) per thread
};

// K unit k of thread tid: unit u = (g * 2 + h) * 64 + 16 r + i is the dword of 8 codes of block g,
// lane group r, of token 16 h + i of the step, the A-operand piece of lane 16 r + i for the tokens
// 16 h .. 16 h + 15 of v_mfma_i32_16x16x32_i8.  The Hadamard layout pairs blocks 2 j and 2 j + 1 in
// one thread (units k, k + 1), so that its producer writes, and its consumers read, both pieces of a
// v_mfma_i32_16x16x64_i8 operand as 16 contiguous bytes at (128 j + 64 h + lane) * 16.
template <int L>
__device__ __forceinline__ int k_unit(int tid, int k) {
  if (L != HAD) return tid + 256 * k;
  const int j = (tid >> 7) + 2 * (k >> 1);
  return ((2 * j + (k & 1)) * 2 + ((tid >> 6) & 1)) * 64 + (tid & 63);
}

// Loaded (not yet unpacked) inputs of one step, per thread.
template <int L, int D>
struct PLoad {
  uint32_t kw[PStep<L, D>::KU];     // K payload dword of each K unit
  uint32_t kh[PStep<L, D>::KU];     // q6_0: the unit's 16 bits of top-bit pairs; q8_0: its second dword
  uint32_t vb[PStep<L, D>::VU][8];  // V payload byte (q8_0: the two bytes) of elements (d, d+1) of each token
  uint32_t vh[PStep<L, D>::VU][8];  // q6_0: the byte of top-bit pairs of (d, d+1)
  uint32_t vs[PStep<L, D>::VU][8];  // V record word of the group of d (zeroed past the end)
  uint32_t kr;                      // one dword of the K records
  uint32_t vr;                      // Hadamard layout: the V scale of token tid (tid < 32)
};

// Raw steps reach LDS by direct loads (the decode's staging layout: a K slot and a V slot per
// step, see Step), NR steps ahead; the block then reads each step's inputs from LDS.
template <int L, int D>
struct PrefillShape {
  using ST = Step<L, D, true>;
  static constexpr int OPS = 2 * PStep<L, D>::BYTES;        // the two operand buffers
  static constexpr int BUDGET = 81920;                          // two blocks per CU
  static constexpr int NR_FIT = (BUDGET - OPS) / (2 * ST::HALF);
  static constexpr int NR = NR_FIT < 2 ? 2 : (NR_FIT > 6 ? 6 : NR_FIT);
  static constexpr int LDS = OPS + NR * 2 * ST::HALF;
};

// One step's inputs for this thread from its raw slot (K slot, V slot), in the units the
// producer works on.
template <int L, int D>
__device__ __forceinline__ void prefill_fetch(const unsigned char* kslot, const unsigned char* vslot, int tid,
                                              PLoad<L, D>& ld) {
  using T = Layout<L, D>;
  using PS = PStep<L, D>;
  using ST = Step<L, D, true>;
  constexpr int PB = T::PB, SB = T::SB;
#pragma unroll
  for (int k = 0; k < PS::KU; ++k) {
    const int u = k_unit<L>(tid, k);
    const int i = u & 15, r = (u >> 4) & 3, h = (u >> 6) & 1, g = u >> 7;
    const int t = 16 * h + i;
    if (L == Q60) {
      const unsigned char* row = kslot + ST::KP + t * PB;
      ld.kw[k] = *reinterpret_cast<const uint32_t*>(row + 24 * g + 4 * r);
      ld.kh[k] = *reinterpret_cast<const uint16_t*>(row + 24 * g + 16 + 2 * r);
    } else if (L == Q80) {
      const uint2 w = *reinterpret_cast<const uint2*>(kslot + ST::kbytes8(t, g, r));
      ld.kw[k] = w.x;
      ld.kh[k] = w.y;
    } else {
      ld.kw[k] = *reinterpret_cast<const uint32_t*>(kslot + ST::kword(t, g, r));
    }
  }
#pragma unroll
  for (int k = 0; k < PS::VU; ++k) {
    const int u = tid + 256 * k;
    const int dp8 = u & 7, r = (u >> 3) & 3, dt = u >> 5;
    const int d = 16 * dt + 2 * dp8;           // even element; the unit covers d and d + 1
    const int g = d >> 5;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int t = 16 * (s >> 2) + 4 * r + (s & 3);
      if (L == Q60) {
        const unsigned char* vrow = vslot + ST::VP + t * PB;
        const int e = d & 31;
        ld.vb[k][s] = vrow[24 * g + (e >> 1)];
        ld.vh[k][s] = vrow[24 * g + 16 + (e >> 2)];
      } else if (L == Q80) {
        ld.vb[k][s] = *reinterpret_cast<const uint16_t*>(vslot + ST::vbytes8(t, d >> 3) + (d & 7));
      } else {   // the byte of elements (d, d + 1): one byte read, the byte index in the address
        ld.vb[k][s] = vslot[ST::vword(t, d >> 3) + ((d >> 1) & 3)];
      }
      const unsigned char* rec = vslot + ST::VR + t * SB;
      if (L == HAD) ld.vs[k][s] = 0u;   // its scales go to VR (ld.vr)
      else if (L == ASYM) ld.vs[k][s] = *reinterpret_cast<const uint32_t*>(rec + 4 * g);
      else ld.vs[k][s] = *reinterpret_cast<const uint16_t*>(rec + 2 * g);
    }
  }
  ld.kr = *reinterpret_cast<const uint32_t*>(kslot + ST::KR + 4 * (tid < 8 * SB ? tid : 0));
  if (L == HAD) ld.vr = *reinterpret_cast<const uint32_t*>(vslot + ST::VR + 4 * (tid & 31));
}

// Unpack and dequantise the loaded step into the LDS buffer.
// n_tok: tokens of the step inside the chunk; the V scales of the others are zeroed so that their
// (stale) rows contribute exact zeros.  The Hadamard layout's V^T holds the codes themselves (exact
// in fp16) and its f32 scales go to VR for the consumers.
// rsign: XORed into every K record dword (the sign bits of its scales and offsets when the rows'
// score scale is negative, so that the consumers see the negated scores and scale them by |sqc|).
template <int L, int D>
__device__ __forceinline__ void prefill_produce(unsigned char* buf, int tid, const PLoad<L, D>& ld, int n_tok,
                                                uint32_t magic, uint32_t rsign) {
  using T = Layout<L, D>;
  using PS = PStep<L, D>;
  constexpr int SB = T::SB;
  constexpr int BIAS = CodeBias<L>::value;
  if (L == HAD) {   // k_unit: a thread's units k and k + 1 are blocks g, g + 1 of one (half, lane)
#pragma unroll
    for (int k = 0; k < PS::KU; k += 2) {
      uint32_t c[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        // signed codes c = (c + 8) - 8 per byte (+0x78 never carries out of a byte), so that the
        // Q K^T MFMA needs no block-sum offset
        const uint32_t x = ld.kw[k + e] ^ 0x88888888u;   // two's-complement nibbles: top bit flipped, c + 8
        c[2 * e] = ((x & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
        c[2 * e + 1] = (((x >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
      }
      *reinterpret_cast<u32x4*>(buf + PS::KC + 16 * (tid + 128 * k)) = u32x4{c[0], c[1], c[2], c[3]};
    }
  }
#pragma unroll
  for (int k = 0; k < (L == HAD ? 0 : PS::KU); ++k) {
    const int u = tid + 256 * k;
    uint32_t lo, hi;
    if (L == Q60) {
      q6_octet(ld.kw[k], ld.kh[k], lo, hi);
    } else if (L == Q80) {
      lo = ld.kw[k];
      hi = ld.kh[k];
    } else {
      const uint32_t x = BIAS ? (ld.kw[k] ^ 0x88888888u) : ld.kw[k];
      lo = x & 0x0F0F0F0Fu;
      hi = (x >> 4) & 0x0F0F0F0Fu;
    }
    *reinterpret_cast<uint2*>(buf + PS::KC + 8 * u) = make_uint2(lo, hi);
  }
#pragma unroll
  for (int k = 0; k < PS::VU; ++k) {
    const int u = tid + 256 * k;
    const int dp8 = u & 7, r = (u >> 3) & 3, dt = u >> 5;
    const int d = 16 * dt + 2 * dp8;
    h2 lowv[4], highv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // tokens of slots 2i and 2i + 1 side by side: [byte(2i), 0, byte(2i + 1), 0]
      const uint32_t y = __builtin_amdgcn_perm(ld.vb[k][2 * i + 1], ld.vb[k][2 * i], 0x0C040C00u);
      uint32_t c0, c1;   // element d and d + 1 of both tokens, as code + bias
      if (L == Q80) {
        c0 = y ^ 0x00800080u;
        c1 = __builtin_amdgcn_perm(ld.vb[k][2 * i + 1], ld.vb[k][2 * i], 0x0C050C01u) ^ 0x00800080u;
      } else if (L == Q60) {
        const int sh = 2 * (d & 3);
        const uint32_t hy = __builtin_amdgcn_perm(ld.vh[k][2 * i + 1], ld.vh[k][2 * i], 0x0C040C00u) >> sh;
        c0 = ((y & 0x000F000Fu) | ((hy & 0x00030003u) << 4)) ^ 0x00200020u;
        c1 = (((y >> 4) & 0x000F000Fu) | ((hy & 0x000C000Cu) << 2)) ^ 0x00200020u;
      } else {
        const uint32_t yb = BIAS ? (y ^ 0x00880088u) : y;
        c0 = yb & 0x000F000Fu;
        c1 = (yb >> 4) & 0x000F000Fu;
      }
      const h2 off = h2{(_Float16)(1024 + BIAS), (_Float16)(1024 + BIAS)};
      h2 v0 = as_h2(c0 | magic) - off;
      h2 v1 = as_h2(c1 | magic) - off;
      const int r4 = 4 * ((u >> 3) & 3);
      const int t0 = 16 * (i >> 1) + r4 + 2 * (i & 1);     // tokens of slots 2i and 2i + 1
      const uint32_t w0 = t0 < n_tok ? ld.vs[k][2 * i] : 0u;
      const uint32_t w1 = t0 + 1 < n_tok ? ld.vs[k][2 * i + 1] : 0u;
      if (L != HAD) {
        const h2 s2 = as_h2(__builtin_amdgcn_perm(w1, w0, 0x05040100u));
        if (L == ASYM) {
          const h2 z2 = as_h2(__builtin_amdgcn_perm(w1, w0, 0x07060302u));
          v0 = v0 * s2 + z2;
          v1 = v1 * s2 + z2;
        } else {
          v0 = v0 * s2;
          v1 = v1 * s2;
        }
      }
      lowv[i] = v0;
      highv[i] = v1;
    }
    unsigned char* dst = buf + PS::VT + (((dt * 4 + r) * 16) + (d & 15)) * 16;
    *reinterpret_cast<u32x4*>(dst) = u32x4{as_u32(lowv[0]), as_u32(lowv[1]), as_u32(lowv[2]), as_u32(lowv[3])};
    *reinterpret_cast<u32x4*>(dst + 16) =
        u32x4{as_u32(highv[0]), as_u32(highv[1]), as_u32(highv[2]), as_u32(highv[3])};
  }
  if (tid < 8 * SB) *reinterpret_cast<uint32_t*>(buf + PS::KR + 4 * tid) = ld.kr ^ rsign;
  if (L == HAD && tid < 32) *reinterpret_cast<uint32_t*>(buf + PS::VR + 4 * tid) = tid < n_tok ? ld.vr : 0u;
}

// Lazy running maximum: a row's maximum is raised, and its l and accumulators rescaled, only when a
// step's scores pass it by more than kLazyMax (log2 units).  Until then the row's probabilities lie in
// [0, 2^kLazyMax], which the f16 P operand holds at its full relative precision; l and the accumulators
// are all relative to the same maximum, so the partial (m, l, o) is the same up to rounding whichever
// maximum it carries.  Most steps then skip the rescale of the accumulators.
constexpr float kLazyMax = 8.0f;

// One step of one wave: Q K^T for the wave's TPW tiles of 16 rows, online softmax, P V.  Each V^T
// operand read from LDS serves every tile of the wave.
// FULL: all 32 tokens exist and every row of the wave sees them.
// Scores: xs holds them unscaled (the i32 dots times the K scales; the Hadamard layout's K codes are
// staged signed, so its dots carry no block-sum offset).  The row's scale sqa = |sqc| > 0 is applied in the
// exponent, exp2(x sqa - m) in one fma, and scaling the step's maximum by sqa keeps the order; a
// negative sqc is carried by the K records, whose signs the producer flipped.
// e_run: Hadamard layout, the wave's V-scale exponent (vscale_exp); the accumulators are in units of
// 2^e_run and P carries p * s_v / 2^e_run.
template <int L, int D, bool FULL, int TPW>
__device__ __forceinline__ void prefill_consume(const unsigned char* buf, int lane, int T0, int n_tok, const int* lim,
                                                const v4i (*qb)[(D / 32 + 1) / 2], const float (*qsB)[(D / 32 + 3) / 4],
                                                const int* qoff0, const float* sqa, float* m_run, float* l_run,
                                                int& e_run, v4f (*oacc)[D / 16]) {
  using T = Layout<L, D>;
  using PS = PStep<L, D>;
  constexpr int NG = T::NG, SG = T::SG, SB = T::SB;
  const int col = lane & 15, r = lane >> 4;
  // Q K^T one tile after the other (its accumulators die with the tile's scores); the K codes are
  // read again for the second tile, which costs less than keeping both tiles' accumulators live
  float xs[TPW][8];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      v4i acc[SG];
      if (L == HAD) {
        // one scale per token: two 32-code groups per v_mfma_i32_16x16x64_i8, the groups' 8-byte
        // operand pieces side by side in A and in B (the same pairing of bytes on both sides, so the
        // integer sum is that of two 16x16x32 products)
#pragma unroll
        for (int g = 0; g < NG; g += 2) {
          const v4i A = *reinterpret_cast<const v4i*>(buf + PS::KC + (((g >> 1) * 2 + tau) * 64 + lane) * 16);
          acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, qb[u][g / 2], g == 0 ? v4i{0, 0, 0, 0} : acc[0], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const uint2 w = *reinterpret_cast<const uint2*>(buf + PS::KC + ((g * 2 + tau) * 64 + lane) * 8);
          const long A = (long)((uint64_t)w.x | ((uint64_t)w.y << 32));
          const v4i q2 = qb[u][g / 2];
          const long B = __builtin_bit_cast(long, (g & 1) ? u32x2{(unsigned)q2[2], (unsigned)q2[3]}
                                                          : u32x2{(unsigned)q2[0], (unsigned)q2[1]});
          acc[g] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, v4i{0, 0, 0, 0}, 0, 0, 0);
        }
      }
      v4f xo = v4f{0.f, 0.f, 0.f, 0.f};
      if (L != HAD && L != Q80) {   // the 8-bit K codes carry no offset
        // offset term sum_g c_g(t) qsum_g: A[t = col][k = r] from the record of token 16 tau + col
        const unsigned char* orec = buf + PS::KR + (16 * tau + col) * SB;
#pragma unroll
        for (int i = 0; i < NG / 4; ++i) {
          const _Float16* h = reinterpret_cast<const _Float16*>(orec);
          const float av = (L == ASYM) ? (float)h[2 * (4 * i + r) + 1] : (float)h[4 * i + r];
          xo = __builtin_amdgcn_mfma_f32_16x16x4f32(av, qsB[u][i], xo, 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tl = 16 * tau + 4 * r + j;
        const unsigned char* rec = buf + PS::KR + tl * SB;
        const bool vis = FULL || (tl < n_tok && T0 + tl <= lim[u]);
        float x;
        if (L == HAD) {
          x = (float)acc[0][j] * *reinterpret_cast<const float*>(rec);   // signed codes: no offset
        } else {
          x = xo[j];
#pragma unroll
          for (int g = 0; g < SG; ++g) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(rec)[(L == ASYM) ? g : (g >> 1)];
            const float sc = (float)as_h2(w)[(L == ASYM) ? 0 : (g & 1)];
            x = fmaf(sc, (float)acc[g][j], x);
          }
        }
        xs[u][tau * 4 + j] = vis ? x : -INFINITY;
      }
    }
  }

  // Hadamard layout: the V scales of the lane's 8 tokens (16 tau + 4 r + j); the exponent of the
  // largest so far grows only where one of them reaches 2^e_run.  A rescale is needed only where a
  // step's scaled score passes its row's maximum by kLazyMax or where the exponent grows: each lane
  // tests its own 8 tokens (a row's maximum passes the bound exactly when the lane holding it does),
  // and the row maxima and the exponent, which need cross-lane steps, are formed in the wave's one
  // branch, as they were in every step before.
  float vsc[8];
  int e_new = e_run;
  float vmax = 0.0f;
  v4f a0, a1;
  bool up = false;
  if (L == HAD) {
    a0 = *reinterpret_cast<const v4f*>(buf + PS::VR + 16 * r);
    a1 = *reinterpret_cast<const v4f*>(buf + PS::VR + 64 + 16 * r);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vmax = fmax_pos(vmax, fmax_pos(a0[j], a1[j]));   // scales >= 0
    }
    up = vscale_exp(vmax) > e_run;
  }
  float smx[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    float smax = xs[u][0];
#pragma unroll
    for (int i = 1; i < 8; ++i) smax = fmaxf(smax, xs[u][i]);
    smx[u] = smax;
    up = up || smax * sqa[u] > m_run[u] + kLazyMax;   // -inf * sqa stays -inf (sqa > 0)
  }
  if (__builtin_amdgcn_ballot_w64(up) != 0) {
    if (L == HAD) e_new = max(e_run, vscale_exp(max_over_rows(vmax)));
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const float smax = max_over_rows(smx[u]);
      const float sm = smax == -INFINITY ? -INFINITY : smax * sqa[u];
      const float m_new = sm > m_run[u] + kLazyMax ? sm : m_run[u];
      // exactly 1 where the maximum held; 0 from an empty row (-inf) to a finite maximum
      const float corr = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[u] - m_new);
      l_run[u] *= corr;
      const float ocorr = L == HAD ? __builtin_amdgcn_ldexpf(corr, e_run - e_new) : corr;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) oacc[u][i] *= ocorr;
      m_run[u] = m_new;
    }
  }
  e_run = e_new;
  if (L == HAD) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vsc[j] = __builtin_amdgcn_ldexpf(a0[j], -e_new);
      vsc[4 + j] = __builtin_amdgcn_ldexpf(a1[j], -e_new);
    }
  }
  v8h pB[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const float nm = m_run[u] == -INFINITY ? 0.0f : -m_run[u];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(xs[u][i], sqa[u], nm));
      psum += p;
      pB[u][i] = (_Float16)(L == HAD ? p * vsc[i] : p);
    }
    l_run[u] += psum;
  }

#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const v8h A = *reinterpret_cast<const v8h*>(buf + PS::VT + (dt * 64 + lane) * 16);
#pragma unroll
    for (int u = 0; u < TPW; ++u) oacc[u][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pB[u], oacc[u][dt], 0, 0, 0);
  }
}

// f32 rows of a prefill (the window's newest positions, and for the full-precision prefill the chunk's
// own rows after them), by the block's four waves together: each wave holds a tile of 16 rows (rows
// trow .. trow + nv - 1, run = false when it has none to compute) and the block walks the 16-token
// tiles k0 .. kend - 1 of the f32 rows once, staging each tile's K and V in LDS for all four waves by
// direct loads issued one tile ahead (one barrier per tile), instead of every wave reading them for
// itself.  Per wave the arithmetic is window_wave's with the operands of Q K^T swapped, so that the
// scores come out as S[token][row] and P stays in registers: lane (col, r) holds row col against tokens
// 4 r + j, which is the A operand of the P V MFMA that takes tokens 4 r + j (k = r); the softmax keeps a
// lazy maximum per row.
// The block's tiles end at the farthest limit of its rows (lmax_blk); a wave computes only up to its
// own rows'.  Every wave of the block calls this with the same k0, kend and lmax_blk.  The rows come
// prepared (a.qrot: the f32 query, rotated for the Hadamard layout).
// Staged tiles, unpadded (direct loads fill 1 KiB runs), in 16-byte chunks swizzled by token t: K chunk x
// of token t at chunk x ^ (t & 15) of its row (a quarter-wave's float4 reads, 16 tokens, then fall on
// distinct banks), V chunk x at x ^ 4 ((t >> 2) & 3) (the four token rows 4 r + j of a P V read start 16
// banks apart).
// Tokens past the last f32 row load the last row instead: their scores are masked and their P is 0.
template <int D>
struct F32Tiles {
  static constexpr int TILE = 16 * D;                   // floats of a K (or V) tile
  static constexpr int K0 = 0, V0 = 2 * TILE;         // float offsets: K, V double buffers
  static constexpr int FLOATS = 4 * TILE;
  static constexpr int BYTES = 4 * FLOATS;
  static constexpr int INSTR = TILE * 4 / 1024 / 4;     // direct loads of a tile per wave
};
template <int D>
__host__ __device__ constexpr int f32_block_lds() { return F32Tiles<D>::BYTES; }

template <int L, int D>
__device__ __forceinline__ void f32_rows_block(const AttendArgs& a, unsigned char* smem, int b, int hk, int S, int trow,
                                               int nv, bool run, int qs0, int k0, int kend, int lmax_blk,
                                               WinState<D>& st) {
  using FT = F32Tiles<D>;
  constexpr int NI = D / 4, CH = D / 4;   // MFMAs of Q K^T; 16-byte chunks of a row
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, r = lane >> 4;
  float* const lds = reinterpret_cast<float*>(smem);
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  const int nrows = a.n_q * a.G;
  const int W = min(S, a.n_recent);
  const int w0 = S - W;
  const int NT = W + (a.kchunk ? a.n_q : 0);
  const size_t ring0 = ((size_t)b * a.Hkv + hk) * a.n_recent;
  // chunk row t - W at cbase + (t - W) cstride floats; ring slot of token t < W: (w0 + t) mod n_recent,
  // the window's positions being consecutive: wr0 + t, less n_recent once it wraps
  const size_t cbase = ((size_t)b * a.n_q * a.Hkv + hk) * D;
  const size_t cstride = (size_t)a.Hkv * D;
  const int wr0 = a.n_recent > 0 ? w0 % a.n_recent : 0;
  const float cl = a.alpha * KVQ_LOG2E;
  if (!run) nv = 0;
  float q[NI];   // the prepared f32 query of row col, elements NI r ..
  {
    const bool ok = col < nv;
    const float* qr = a.qrot + (ok ? row_index(a, b, hk, trow + col) * D : 0) + NI * r;
#pragma unroll
    for (int i = 0; i < NI; i += 4) {
      const float4 v = ok ? *reinterpret_cast<const float4*>(qr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
      q[i] = v.x;
      q[i + 1] = v.y;
      q[i + 2] = v.z;
      q[i + 3] = v.w;
    }
  }
  const int limc = col < nv ? row_limit(a, qs0, trow + col, nrows) : -1;   // row col's last visible position
#pragma unroll
  for (int i = 0; i < D / 16; ++i) st.o[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lrow = 0.0f;   // row col: running maximum, and the sum over this lane's tokens
  auto tiles_to = [&](int lmax) {   // tiles up to the farthest limit lmax (none below the first f32 row)
    int n = min((NT + 15) / 16, kend);
    if (lmax < w0) n = 0;
    else if ((lmax - w0) / 16 + 1 < n) n = (lmax - w0) / 16 + 1;
    return n;
  };
  const int nt_wave = tiles_to(nv > 0 ? row_limit(a, qs0, trow + nv - 1, nrows) : -1);
  const int nt_blk = tiles_to(lmax_blk);
  // Direct loads of tile k into buffer k & 1: this wave's instructions n = INSTR w .. INSTR w + INSTR - 1
  // of each of K and V, lane l of instruction n filling chunk position p = 64 n + l (token p / CH).
  auto issue = [&](int k) {
#pragma unroll
    for (int i = 0; i < FT::INSTR; ++i) {
      const int n = FT::INSTR * wave + i;
      const int p = 64 * n + lane;
      const int tok = p / CH, x = p % CH;
      const int t = min(16 * k + tok, NT - 1);
      const float* ksrc;
      const float* vsrc;
      if (t >= W) {
        const size_t co = cbase + (size_t)(uint32_t)(t - W) * cstride;
        ksrc = a.kchunk + co;
        vsrc = a.vchunk + co;
      } else {
        const int slot = wr0 + t >= a.n_recent ? wr0 + t - a.n_recent : wr0 + t;
        const size_t ro = (ring0 + (size_t)slot) * D;
        ksrc = a.kring + ro;
        vsrc = a.vring + ro;
      }
      const uint32_t kb = lds_base + 4 * (FT::K0 + (k & 1) * FT::TILE) + 1024 * n;
      const uint32_t vb = lds_base + 4 * (FT::V0 + (k & 1) * FT::TILE) + 1024 * n;
      dma16(reinterpret_cast<const uint8_t*>(ksrc + 4 * (x ^ (tok & 15))), kb);
      dma16(reinterpret_cast<const uint8_t*>(vsrc + 4 * (x ^ (4 * ((tok >> 2) & 3)))), vb);
    }
  };
  if (k0 < nt_blk) issue(k0);
  wait_vm<0>();
  __syncthreads();
  for (int k = k0; k < nt_blk; ++k) {
    if (k + 1 < nt_blk) issue(k + 1);
    if (k < nt_wave) {
      const float* kt = lds + FT::K0 + (k & 1) * FT::TILE;
      const float* vt = lds + FT::V0 + (k & 1) * FT::TILE;
      // ---- S^T = K Q^T: lane (col, r) supplies K of token col (A) and Q of row col (B), elements NI r + i
      // in MFMA i; it then holds S[token 4 r + j][row col]
      v4f c = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NI; i += 4) {
        const int x = (NI * r + i) / 4;
        const float4 kv = *reinterpret_cast<const float4*>(kt + col * D + 4 * (x ^ col));
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.x, q[i], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.y, q[i + 1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.z, q[i + 2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.w, q[i + 3], c, 0, 0, 0);
      }
      // ---- online softmax of row col over the tile's 16 tokens (four per lane), with a lazy maximum:
      // the row's maximum, and its l and accumulators, change only in a tile where one of its scores
      // passes it by kLazyMax (each lane tests its own tokens; one branch for the wave), so p lies in
      // [0, 2^8]
      float xs[4];
      bool up = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tj = 16 * k + 4 * r + j;
        xs[j] = (tj < NT && w0 + tj <= limc) ? c[j] * cl : -INFINITY;
        up = up || xs[j] > mrow + kLazyMax;
      }
      if (__builtin_amdgcn_ballot_w64(up) != 0) {
        float mx = fmax_nc(fmax_nc(xs[0], xs[1]), fmax_nc(xs[2], xs[3]));
        mx = fmax_nc(mx, __shfl_xor(mx, 16));   // the row's four lane groups
        mx = fmax_nc(mx, __shfl_xor(mx, 32));
        const float m_new = fmax_nc(mrow, mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float corr = __builtin_amdgcn_exp2f(mrow - m_use);   // results below 2^-126 (against a maximum of 1)
        lrow *= corr;
        mrow = m_new;
        // the accumulators hold rows 4 r + j: their corrections come from lanes 4 r + j
        float cj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) cj[j] = __shfl(corr, 4 * r + j);
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          v4f o = st.o[i];
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] *= cj[j];
          st.o[i] = o;
        }
      }
      const float m_use = mrow == -INFINITY ? 0.0f : mrow;
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(xs[j] - m_use);   // may flush: they change no sum
        lrow += p[j];
      }
      // ---- P V: MFMA j takes tokens 4 r + j (k = r), A = P[row col][token 4 r + j] from this lane
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* vrow = vt + (4 * r + j) * D;   // token 4 r + j: swizzle 4 r
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const int e = col + 16 * dt;
          st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[j], vrow[4 * ((e >> 2) ^ (4 * r)) + (e & 3)], st.o[dt], 0, 0, 0);
        }
      }
    }
    wait_vm<0>();        // this wave's loads of tile k + 1 have landed
    __syncthreads();     // every wave's have, and every wave is done with buffer k & 1
  }
  // the state of rows 4 r + j, as the accumulators hold them: l summed over the row's four lane groups
  lrow += __shfl_xor(lrow, 16);
  lrow += __shfl_xor(lrow, 32);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    st.m[j] = __shfl(mrow, 4 * r + j);
    st.l[j] = __shfl(lrow, 4 * r + j);
  }
}

// Grid: one block per (batch row, kv head, group, block of BR rows), the groups being the chunks of
// the quantised region and then a.nwg groups of f32 rows (window, chunk rows; a prefill without
// packed chunks runs them through prefill_rows_f32 instead).  Each wave takes TPW consecutive
// 16-row tiles of the block (two at head_dim 128, so that the block's shared unpacking and
// dequantisation serve 128 rows; one at 256 and for q6_0, where the registers would not hold it).
// The rows' int8 queries, scales and block sums come prepared by prepare_rows.
template <int L, int D>
struct PrefillTiles {
  static constexpr int TPW = (D == 128 && L != Q60) ? 2 : 1;   // 16-row tiles per wave
  static constexpr int BR = 64 * TPW;                          // rows per block
  // blocks per CU: three for the Hadamard layout at head_dim 128, whose registers (168 under this
  // bound) and LDS allow it, two for the others
  static constexpr int OCC = (L == HAD && D == 128) ? 3 : 2;
};
static_assert(PrefillTiles<HAD, 128>::OCC * PrefillShape<HAD, 128>::LDS <= 160 * 1024 &&
                  PrefillTiles<HAD, 128>::OCC * f32_block_lds<128>() <= 160 * 1024,
              "three Hadamard head_dim-128 prefill blocks per CU");

template <int L, int D>
__global__ __launch_bounds__(256, (PrefillTiles<L, D>::OCC)) void prefill_partial(AttendArgs a) {
  using T = Layout<L, D>;
  using PS = PStep<L, D>;
  constexpr int NG = T::NG;
  constexpr int BIAS = CodeBias<L>::k_side;
  constexpr int TPW = PrefillTiles<L, D>::TPW, BR = PrefillTiles<L, D>::BR;
  extern __shared__ __align__(16) unsigned char smem[];

  // One-dimensional grid in an XCD-aware order: the chip hands consecutive blocks round robin to
  // its 8 XCDs (block id runs on XCD id % 8), so virtual index v gives each XCD a contiguous
  // range, and v puts the row blocks of one (batch row, kv head, chunk) next to each other:
  // they read the same K/V, which their XCD's L2 then holds for all of them.
  const int nrb = (a.n_q * a.G + BR - 1) / BR;
  const int id = (int)blockIdx.x, nblocks = (int)gridDim.x;
  const int v = (nblocks % 8 == 0) ? (id % 8) * (nblocks / 8) + id / 8 : id;
  const int rb = v % nrb;
  const int rest = v / nrb;
  const int c = rest % a.ngroups;
  const int hk = (rest / a.ngroups) % a.Hkv, b = rest / a.ngroups / a.Hkv;
  const int S = a.seq_len[b];
  const int Sq = a.n_recent > 0 ? max(0, S - a.n_recent) : S;
  const int nrows = a.n_q * a.G;
  const int row0 = BR * rb;
  const int nblk = min(BR, nrows - row0);
  const int qs0 = a.causal ? a.q_start[b] : 0;
  // the last a.nwg groups of this grid (if any): f32 rows (the window; for the full-precision prefill
  // also the chunk's own rows, in a.nwin slices of a.slice rows)
  const int nch = a.ngroups - a.nwg;
  if (c >= nch) {   // f32-row block: wave w takes the 16-row tiles TPW w .. TPW w + TPW - 1, one per pass
    const int w = threadIdx.x >> 6;
    const int j = c - nch;
    const int k0 = a.kchunk ? j * (a.slice / 16) : 0;
    const int kend = a.kchunk ? k0 + a.slice / 16 : 0x7fffffff;
    const int lmax_blk = nblk > 0 ? row_limit(a, qs0, row0 + nblk - 1, nrows) : -1;
#pragma unroll 1
    for (int u = 0; u < TPW; ++u) {
      const int trow = row0 + 16 * (TPW * w + u);
      const int nv = min(16, nblk - 16 * (TPW * w + u));
      bool run = (S > 0 || a.kchunk) && nv > 0;
      if (a.kchunk && run) {   // a slice past every limit of the tile's rows: the reduce does not read it
        const int lmax = row_limit(a, qs0, trow + nv - 1, nrows);
        run = j * a.slice <= lmax - (S - min(S, a.n_recent));
      }
      WinState<D> st;
      f32_rows_block<L, D>(a, smem, b, hk, S, trow, nv, run, qs0, k0, kend, lmax_blk, st);   // every wave
      if (run) window_store<D>(a, st, b, hk, trow, nv, threadIdx.x & 63, a.nc1 - a.nwin + j);
    }
    return;
  }
  const int t_begin = c * a.chunk;
  if (t_begin >= Sq) return;
  int t_end = min(t_begin + a.chunk, Sq);
  const int lim_blk = row_limit(a, qs0, row0 + nblk - 1, nrows);
  if (a.skip && lim_blk < t_end - 1) t_end = max(t_begin, lim_blk + 1);   // causal skip
  const int nsteps = (t_end - t_begin + 31) / 32;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, r = lane >> 4;
  const int wrow0 = row0 + 16 * TPW * wave;            // the wave's first row
  int nval[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) nval[u] = min(16, max(0, nblk - 16 * (TPW * wave + u)));

  // ---- prologue: this wave's rows from the prepared rows (int8 query in the B-operand order, its
  // scale and block sums); the perms consume the loads here, outside the streaming loop
  constexpr int NQ = (NG + 3) / 4;
  v4i qb[TPW][(NG + 1) / 2];   // group g's 8 bytes: elements 2 (g & 1), 2 (g & 1) + 1 of qb[u][g / 2]
  float qsB[TPW][NQ];
  int qoff0[TPW], lim[TPW];
  float sqa[TPW];   // |score scale| in log2 units, at least FLT_MIN (so that -inf * sqa stays -inf)
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int trow = wrow0 + 16 * u;
#pragma unroll
    for (int g = 0; g < (NG + 1) / 2; ++g) qb[u][g] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NQ; ++i) qsB[u][i] = 0.0f;
    qoff0[u] = 0;
    float sqc = 0.0f;
    if (col < nval[u]) {
      const size_t fr = row_index(a, b, hk, trow + col);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const uint2 w = *reinterpret_cast<const uint2*>(a.q8p + fr * D + 32 * g + 8 * r);
        const uint32_t lo = L == Q80 ? w.x : __builtin_amdgcn_perm(w.y, w.x, 0x06040200u);
        const uint32_t hi = L == Q80 ? w.y : __builtin_amdgcn_perm(w.y, w.x, 0x07050301u);
        qb[u][g / 2][2 * (g & 1)] = (int)lo;
        qb[u][g / 2][2 * (g & 1) + 1] = (int)hi;
      }
      const int* qs = a.qsump + fr * NG;
#pragma unroll
      for (int i = 0; i < NG / 4; ++i)
        qsB[u][i] = (L == ASYM) ? (float)qs[4 * i + r] : -(float)BIAS * (float)qs[4 * i + r];
      int tot = 0;
#pragma unroll
      for (int g = 0; g < NG; ++g) tot += qs[g];
      qoff0[u] = BIAS * tot;
      sqc = a.sqp[fr] * a.alpha * KVQ_LOG2E;
    }
    sqa[u] = fmaxf(fabsf(sqc), __FLT_MIN__);
    lim[u] = row_limit(a, qs0, trow + col, nrows);
  }
  const int lim_min = row_limit(a, qs0, wrow0, nrows);   // the wave's smallest limit; -1 without rows

  float m_run[TPW], l_run[TPW];
  int e_run = kNoExp;   // Hadamard layout: the accumulators are in units of 2^e_run
  v4f oacc[TPW][D / 16];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    m_run[u] = -INFINITY;
    l_run[u] = 0.0f;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[u][i] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // a negative score scale (alpha < 0): the K records' signs flipped, so that sqa = |sqc| applies
  const uint32_t rsign = a.alpha < 0.0f ? (L == HAD ? 0x80000000u : 0x80008000u) : 0u;
  uint32_t magic;   // fp16 "1024 + code" exponent bits, in a VGPR so v_and_or_b32 can take it
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  // Raw steps in a ring of NR slots after the two operand buffers, NR - 1 steps ahead: wave 0 loads
  // each step's K half, wave 1 its V half.  Iteration s: issue step s + NR - 1 (into the slot step
  // s - 1 left, read two iterations ago), wait for step s + 1, barrier, produce step s + 1 into
  // operand buffer (s + 1) & 1 (read by consume at s - 1, before this barrier), consume step s
  // (produced before it).  The raw loads complete in issue order, so a wave's count of the steps
  // it issued after s + 1 bounds its wait; the barrier then publishes the slot to every wave.
  using PSh = PrefillShape<L, D>;
  using ST = Step<L, D, true>;
  constexpr int NR = PSh::NR, H = ST::HALF, G = ST::GROUP;
  unsigned char* raw = smem + PSh::OPS;
  const uint32_t raw_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)raw);
  auto issue = [&](int st) {
    const uint32_t slot = raw_lds + (st % NR) * 2 * H;
    if (wave == 0) issue_dma_half<ST, false>(a, half_rows_s(a, b, hk, t_begin + 32 * st, t_end), lane, slot);
    else if (wave == 1) issue_dma_half<ST, true>(a, half_rows_s(a, b, hk, t_begin + 32 * st, t_end), lane, slot + H);
  };
  auto wait_steps = [&](int n) {   // this wave's loads of all but the newest n steps have landed
    if (wave < 2) {
      switch (n) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<G>(); break;
        case 2: wait_vm<2 * G>(); break;
        case 3: wait_vm<3 * G>(); break;
        default: wait_vm<4 * G>(); break;
      }
    }
  };
  static_assert(NR - 2 <= 4 && 4 * G <= 63, "load counter range");
  auto raw_k = [&](int st) { return raw + (st % NR) * 2 * H; };
  auto barrier = [] {
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");   // this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" : : : "memory");
  };

  PLoad<L, D> ld;
#pragma unroll
  for (int i = 0; i < NR - 1; ++i)
    if (i < nsteps) issue(i);
  if (nsteps > 0) {
    wait_steps(min(nsteps - 1, NR - 2));
    barrier();
    prefill_fetch<L, D>(raw_k(0), raw_k(0) + H, tid, ld);
    prefill_produce<L, D>(smem, tid, ld, min(32, t_end - t_begin), magic, rsign);
  }
  // Steps whose 32 tokens are all present and visible to every row of the wave come first (the
  // condition only turns from true to false along the chunk): each loop then has one consume form,
  // and the accumulators stay in place instead of being copied at an if/else join every step.
  const int nfull_a = (t_end - t_begin) / 32;
  const int nfull_b = lim_min + 1 - t_begin >= 0 ? (lim_min + 1 - t_begin) / 32 : 0;
  const int nfull = min(min(nfull_a, nfull_b), nsteps);
  // the priority drops after steps p2, p1, p0: the first s with 8 (s + 1) >= 4, 6, 7 nsteps
  const int p2 = (4 * nsteps + 7) / 8 - 1, p1 = (6 * nsteps + 7) / 8 - 1, p0 = (7 * nsteps + 7) / 8 - 1;
  auto step = [&](int s, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int T0 = t_begin + 32 * s;
    const bool more = s + 1 < nsteps;
    if (s + NR - 1 < nsteps) issue(s + NR - 1);
    if (s + NR - 1 < nsteps) {   // steady part: a constant count, without wait_steps' branches
      if (wave < 2) wait_vm<(NR - 2) * G>();
    } else if (more) {
      wait_steps(nsteps - 1 - (s + 1));
    }
    barrier();
    if (more) {
      prefill_fetch<L, D>(raw_k(s + 1), raw_k(s + 1) + H, tid, ld);
      prefill_produce<L, D>(smem + ((s + 1) & 1) * PS::BYTES, tid, ld, min(32, t_end - T0 - 32), magic, rsign);
    }
    const unsigned char* buf = smem + (s & 1) * PS::BYTES;
    const int n_tok = min(32, t_end - T0);
    if (nval[0] > 0)
      prefill_consume<L, D, FULL, TPW>(buf, lane, T0, n_tok, lim, qb, qsB, qoff0, sqa, m_run, l_run, e_run, oacc);
    // Issue priority by progress, as in the decode kernel: a SIMD's waves come from different blocks of
    // equal work and would otherwise finish oldest first (causal prefill 110 -> 106 us).  Not in the
    // full-precision prefill, whose f32-row blocks at the end of the grid then waited behind the
    // packed blocks (151 -> 156 us with it).
    if (!a.kchunk) {
      if (s == p2) __builtin_amdgcn_s_setprio(2);
      if (s == p1) __builtin_amdgcn_s_setprio(1);
      if (s == p0) __builtin_amdgcn_s_setprio(0);
    }
  };
  if (!a.kchunk) __builtin_amdgcn_s_setprio(3);
  int s = 0;
  for (; s < nfull; ++s) step(s, std::integral_constant<bool, true>{});
  for (; s < nsteps; ++s) step(s, std::integral_constant<bool, false>{});

  // ---------------- this wave's chunk partials (narrow records): o[d = 16 dt + 4 r + j] of row col of
  // each tile, lanes col, col + 16, col + 32 and col + 48 holding the row
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const float l = sum_over_rows(l_run[u]);
    float amax = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) amax = fmax_pos(amax, fabsf(oacc[u][dt][j]));
    amax = fmax_pos(amax, __shfl_xor(amax, 16));
    const int x = narrow_exp(fmax_pos(amax, __shfl_xor(amax, 32)));
    if (col < nval[u]) {
      float* dst = a.ws + (row_index(a, b, hk, wrow0 + 16 * u + col) * a.nc1 + c) * narrow_stride(D);
      uint32_t* hw = reinterpret_cast<uint32_t*>(dst);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const v4f o = oacc[u][dt];
        *reinterpret_cast<u32x2*>(hw + 8 * dt + 2 * r) = u32x2{narrow_pk(o[0], o[1], x), narrow_pk(o[2], o[3], x)};
      }
      if (r == 0) {
        dst[D / 2] = m_run[u];
        dst[D / 2 + 1] = l;
        // the accumulators' unit 2^e_run (Hadamard layout) times the record's scale
        reinterpret_cast<int*>(dst)[D / 2 + 2] = (L == HAD ? e_run : 0) + x - 15;
      }
    }
  }
}

// The f32 rows of a full-precision prefill without a cached prefix: its chunk's own rows in a.nwin
// slices of a.slice rows.  A launch of its own, which needs fewer registers than prefill_partial and
// runs at a higher occupancy (with packed chunks to stream, the f32 rows instead share
// prefill_partial's grid, whose tail they fill).  Grid: one block per (batch row, kv head,
// slice, block of 64 rows), in the XCD-aware order of prefill_partial; wave w takes the 16-row
// tile 16 w of the block.
template <int L, int D>
__global__ __launch_bounds__(256, D == 128 ? 3 : 2) void prefill_rows_f32(AttendArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nrb = (a.n_q * a.G + 63) / 64;
  const int id = (int)blockIdx.x, nblocks = (int)gridDim.x;
  const int v = (nblocks % 8 == 0) ? (id % 8) * (nblocks / 8) + id / 8 : id;
  const int rb = v % nrb;
  const int rest = v / nrb;
  const int j = rest % a.nwin;
  const int hk = (rest / a.nwin) % a.Hkv, b = rest / a.nwin / a.Hkv;
  const int S = a.seq_len[b];
  const int nrows = a.n_q * a.G;
  const int qs0 = a.causal ? a.q_start[b] : 0;
  const int w = threadIdx.x >> 6;
  const int trow = 64 * rb + 16 * w;
  const int nv = min(16, nrows - trow);
  bool run = (S > 0 || a.kchunk) && nv > 0;
  if (a.kchunk && run) {   // a slice past every limit of the tile's rows: the reduce does not read it
    const int lmax = row_limit(a, qs0, trow + nv - 1, nrows);
    run = j * a.slice <= lmax - (S - min(S, a.n_recent));
  }
  const int k0 = a.kchunk ? j * (a.slice / 16) : 0;
  const int kend = a.kchunk ? k0 + a.slice / 16 : 0x7fffffff;
  const int nblk = min(64, nrows - 64 * rb);
  const int lmax_blk = nblk > 0 ? row_limit(a, qs0, 64 * rb + nblk - 1, nrows) : -1;
  WinState<D> st;
  f32_rows_block<L, D>(a, smem, b, hk, S, trow, nv, run, qs0, k0, kend, lmax_blk, st);   // every wave
  if (run) window_store<D>(a, st, b, hk, trow, nv, threadIdx.x & 63, a.nc1 - a.nwin + j);
}

// Finish time of a grid under list scheduling on `slots` identical block slots: n1 blocks of cost w1
// dispatched first, then n2 of cost w2, each block taking the earliest free slot.  Slots are kept
// as (free time, count) groups, so the work is one step per group visited.
static int64_t list_makespan(int64_t slots, int64_t n1, int64_t w1, int64_t n2, int64_t w2) {
  std::map<int64_t, int64_t> free_at{{0, slots}};
  int64_t end = 0;
  auto put = [&](int64_t n, int64_t w) {
    while (n > 0) {
      auto it = free_at.begin();
      const int64_t t = it->first, m = std::min(it->second, n);
      if (it->second > m) it->second -= m;
      else free_at.erase(it);
      free_at[t + w] += m;
      end = std::max(end, t + w);
      n -= m;
    }
  };
  put(n1, w1);
  put(n2, w2);
  return end;
}

// Fixed cost of one prefill block, in packed tokens (its prologue, first loads and partial store),
// and the cost of one f32 row relative to one packed token, for list_makespan.
constexpr int kBlockFixedTokens = 128;
constexpr int kF32RowTokens = 4;

// Split-K chunk of a prefill (a multiple of 32 tokens, at least kPrefillChunk), for row_blocks row
// blocks over `packed` packed tokens (chunks past a row's packed tokens return at once), with
// extra_groups f32-row groups of f32_rows rows each after the chunks.
// The packed blocks may take `cap` of the device's blocks_per_cu x CUs slots: all those the f32-row
// blocks leave when those are light (heavy = false: the causal prefill's window), blocks_per_cu - 1
// per CU when they are heavy (the full-precision prefill's chunk rows, on the f32 MFMA at a sixteenth
// of the f16 rate, which then keep one slot per CU).  The chunk is the shortest whose packed blocks
// fit that cap in one round: on the Hadamard head_dim-128 kernel (three blocks per CU), 512 queries at
// 8192 measured 92 us with 800-token chunks (11 chunks, the rule's choice) against 95-122 with
// 672-1248, and the full-precision prefill 119 us with 1024 (the rule's) against 121-158 with
// 512-2048.  When even one chunk per row block exceeds the cap, the chunk is the one whose grid
// finishes first under list_makespan.
static int prefill_chunk(int64_t row_blocks, int packed, int extra_groups, int f32_rows, bool heavy,
                         int blocks_per_cu) {
  const int64_t slots = (int64_t)blocks_per_cu * device_cus();
  const int64_t cap = heavy ? slots - device_cus() : slots - row_blocks * extra_groups;
  const int kmax = chunks_of(max(packed, 1), kPrefillChunk);
  const int64_t kfit = cap > 0 ? cap / row_blocks : 0;
  if (kfit >= 1) {
    const int k = (int)std::min<int64_t>(kfit, kmax);
    return max(kPrefillChunk, (packed + k - 1) / k + 31) / 32 * 32;
  }
  int best = kPrefillChunk;
  int64_t best_cost = -1;
  // the shortest chunk for each count of chunks with packed tokens, up to four rounds of packed blocks
  for (int k = kmax; k >= 1; --k) {
    const int c = max(kPrefillChunk, (packed + k - 1) / k + 31) / 32 * 32;
    if (k > 1 && (chunks_of(packed, c) != k || row_blocks * k > 4 * slots)) continue;
    const int64_t cost = list_makespan(slots, row_blocks * k, c + kBlockFixedTokens, row_blocks * extra_groups,
                                       (int64_t)kF32RowTokens * f32_rows + kBlockFixedTokens);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

static inline int prefill_rows_per_block(int layout, int D) { return (D == 128 && layout != Q60) ? 128 : 64; }
static inline int prefill_blocks_per_cu(int layout, int D) { return (layout == HAD && D == 128) ? 3 : 2; }
static_assert(PrefillTiles<HAD, 128>::BR == 128 && PrefillTiles<Q60, 128>::BR == 64 && PrefillTiles<Q40, 256>::BR == 64,
              "rows per block as the host computes them");
static_assert(PrefillTiles<HAD, 128>::OCC == 3 && PrefillTiles<HAD, 256>::OCC == 2 && PrefillTiles<Q40, 128>::OCC == 2,
              "blocks per CU as the host computes them");

// Query preparation of every row once (a1), 16 rows per block: int8 query, scale, per-block sums,
// and for the Hadamard layout the rotated f32 query the window uses.
template <int L, int D>
__global__ __launch_bounds__(256) void prepare_rows(const float* q, int n_vec, float* qrot, int8_t* q8, float* sq,
                                                    int* qsum) {
  constexpr int NG = D / 32;
  __shared__ __align__(16) float qf[16 * D];
  __shared__ __align__(16) int8_t q8s[16 * D];
  __shared__ float sqs[16];
  __shared__ int qss[16 * NG];
  const int tid = threadIdx.x;
  const int v0 = blockIdx.x * 16;
  const int nv = min(16, n_vec - v0);
  for (int idx = tid; idx < 4 * D; idx += 256) {     // float4 of 16 rows
    const int row = idx / (D / 4);
    const float4 v = row < nv ? reinterpret_cast<const float4*>(q + (size_t)v0 * D)[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4*>(qf)[idx] = v;
  }
  __syncthreads();
  prepare_query_lds<L, D>(qf, q8s, sqs, qss);
  if (L == HAD) {
    for (int idx = tid; idx < 4 * D; idx += 256)
      if (idx / (D / 4) < nv) reinterpret_cast<float4*>(qrot + (size_t)v0 * D)[idx] = reinterpret_cast<const float4*>(qf)[idx];
  }
  for (int idx = tid; idx < D; idx += 256)          // 16-byte pieces of 16 rows
    if (idx / (D / 16) < nv) reinterpret_cast<u32x4*>(q8 + (size_t)v0 * D)[idx] = reinterpret_cast<const u32x4*>(q8s)[idx];
  if (tid < 16 * NG && tid / NG < nv) qsum[(size_t)v0 * NG + tid] = qss[tid];
  if (tid < nv) sq[v0 + tid] = sqs[tid];
}

template <int L, int D>
static void launch_prepare(const float* q, int n_vec, float* qrot, int8_t* q8, float* sq, int* qsum, hipStream_t st) {
  hipLaunchKernelGGL((prepare_rows<L, D>), dim3((n_vec + 15) / 16), dim3(256), 0, st, q, n_vec, qrot, q8, sq, qsum);
}

typedef void (*prepare_fn)(const float*, int, float*, int8_t*, float*, int*, hipStream_t);

static prepare_fn pick_prepare(int layout, int D) {
  // the preparation differs only by the rotation
  return layout == HAD ? (D == 256 ? launch_prepare<HAD, 256> : launch_prepare<HAD, 128>)
                       : (D == 256 ? launch_prepare<Q40, 256> : launch_prepare<Q40, 128>);
}

// f32 = false: the packed chunks (prefill_partial); f32 = true: the f32 rows (prefill_rows_f32).
template <int L, int D>
static void launch_prefill(const AttendArgs& a, dim3 grid, bool f32, hipStream_t st) {
  if (f32) {
    const size_t lds = f32_block_lds<D>();
    if (lds > 65536)
      (void)hipFuncSetAttribute((const void*)prefill_rows_f32<L, D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((prefill_rows_f32<L, D>), grid, dim3(256), lds, st, a);
    return;
  }
  size_t lds = PrefillShape<L, D>::LDS;
  if (a.nwg > 0 && (size_t)f32_block_lds<D>() > lds) lds = f32_block_lds<D>();
  if (lds > 65536)
    (void)hipFuncSetAttribute((const void*)prefill_partial<L, D>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((prefill_partial<L, D>), grid, dim3(256), lds, st, a);
}

typedef void (*prefill_fn)(const AttendArgs&, dim3, bool, hipStream_t);

static prefill_fn pick_prefill(int layout, int D) {
  const int di = D == 256 ? 1 : 0;
  static const prefill_fn tab[kNumLayouts][2] = {
      {launch_prefill<HAD, 128>, launch_prefill<HAD, 256>},
      {launch_prefill<Q40, 128>, launch_prefill<Q40, 256>},
      {launch_prefill<Q60, 128>, launch_prefill<Q60, 256>},
      {launch_prefill<ASYM, 128>, launch_prefill<ASYM, 256>},
      {launch_prefill<Q80, 128>, launch_prefill<Q80, 256>},
  };
  return tab[layout][di];
}


// Workspace of a prefill: the narrow partial records [rows x nslots x (D / 2 + 4)] floats (nslots: the
// chunks and the f32-row slots of that call), then the prepared rows.
static RowPrep prefill_ws(size_t rows, int D, int nslots) {
  return row_prep_layout(rows * (size_t)nslots * narrow_stride(D) * sizeof(float), rows, D);
}

kvq_status launch_prepare_rows(const kvq_cache* c, const float* q, int n_vec, unsigned char* ws, const RowPrep& w,
                               AttendArgs& a, hipStream_t s) {
  a.qrot = c->layout == HAD ? (const float*)(ws + w.qrot) : q;   // the window's f32 query
  a.q8p = (const int8_t*)(ws + w.q8);
  a.sqp = (const float*)(ws + w.sq);
  a.qsump = (const int*)(ws + w.qsum);
  if (n_vec == 0) return KVQ_OK;
  pick_prepare(c->layout, c->head_dim)(q, n_vec, (float*)(ws + w.qrot), (int8_t*)(ws + w.q8), (float*)(ws + w.sq),
                                       (int*)(ws + w.qsum), s);
  return check_launch("query preparation kernel");
}

}  // namespace kvq

using namespace kvq;

extern "C" size_t kvq_prefill_workspace_bytes(int32_t batch, int32_t n_q, int32_t Hq, int32_t D,
                                              int32_t max_seq_len) {
  if (batch < 1 || n_q < 1 || Hq < 1 || (D != 128 && D != 256) || max_seq_len < 0) return 0;
  // the larger of the two prefills' needs: one window slot, or the slices of a full-precision
  // prefill's f32 rows with the largest window
  const int nslots = chunks_of(max_seq_len, kPrefillChunk) + row_slices(512, n_q);
  return prefill_ws((size_t)batch * n_q * Hq, D, nslots).end;
}

extern "C" kvq_status kvq_attend_prefill_causal(const kvq_cache* c, const float* q, float* out, int32_t batch,
                                                int32_t n_q, int32_t Hq, float alpha, int32_t causal,
                                                const int32_t* q_start, const int32_t* block_table,
                                                int32_t max_pages, const int32_t* seq_len, int32_t max_seq_len,
                                                uint32_t flags, void* workspace, size_t ws_bytes, void* stream) {
  kvq_status st = check_attend_args(c, q, batch, Hq, block_table, max_pages, seq_len, max_seq_len);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out must be non-null");
  if (n_q < 1) return fail(KVQ_ERR_INVALID_ARG, "n_q must be >= 1");
  if (causal != 0 && causal != 1) return fail(KVQ_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (causal && !q_start) return fail(KVQ_ERR_INVALID_ARG, "q_start must be non-null when causal");
  if (flags & ~KVQ_PREFILL_NO_CAUSAL_SKIP) return fail(KVQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((int64_t)batch * n_q * Hq > 0x7fffffff) return fail(KVQ_ERR_UNSUPPORTED, "batch * n_q * num_q_heads above 2^31 - 1");
  const size_t need = kvq_prefill_workspace_bytes(batch, n_q, Hq, c->head_dim, max_seq_len);
  if (!workspace || ws_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  const int64_t rbp = ((int64_t)n_q * (Hq / c->num_kv_heads) + prefill_rows_per_block(c->layout, c->head_dim) - 1) /
                      prefill_rows_per_block(c->layout, c->head_dim) * c->num_kv_heads * batch;
  // packed tokens of the longest row: all but its window
  const int chunk = prefill_chunk(rbp, max(0, max_seq_len - c->n_recent), c->n_recent > 0 ? 1 : 0,
                                  min(c->n_recent, max_seq_len), false, prefill_blocks_per_cu(c->layout, c->head_dim));
  AttendArgs a = make_args(c, q, Hq, n_q, alpha, block_table, max_pages, seq_len, max_seq_len, chunk, workspace);
  a.causal = causal;
  a.skip = causal && !(flags & KVQ_PREFILL_NO_CAUSAL_SKIP);
  a.q_start = causal ? q_start : nullptr;
  const int nch = chunks_of(max_seq_len, chunk);
  a.nwg = c->n_recent > 0 ? 1 : 0;   // the window: one group in the same grid
  a.ngroups = nch + a.nwg;
  const int64_t gx = ((int64_t)n_q * a.G + prefill_rows_per_block(c->layout, c->head_dim) - 1) /
                     prefill_rows_per_block(c->layout, c->head_dim) * a.ngroups * c->num_kv_heads * batch;
  if (gx > 0x7fffffff) return fail(KVQ_ERR_UNSUPPORTED, "prefill grid above 2^31 - 1 blocks");
  const int rows = batch * n_q * Hq;
  const RowPrep w = prefill_ws((size_t)rows, c->head_dim, a.nc1);
  if ((st = launch_prepare_rows(c, q, rows, (unsigned char*)workspace, w, a, (hipStream_t)stream)) != KVQ_OK) return st;
  if (gx > 0) {
    pick_prefill(c->layout, c->head_dim)(a, dim3((unsigned)gx), false, (hipStream_t)stream);
    if ((st = check_launch("prefill partial kernel")) != KVQ_OK) return st;
  }
  return launch_reduce(c, out, batch, n_q * Hq, seq_len, a.nc1, chunk, (const float*)workspace,
                       (hipStream_t)stream, 0, 0, 0, RunSplit{}, true);
}

extern "C" kvq_status kvq_prefill_full_then_store(const kvq_cache* c, const float* q, const float* k_new,
                                                  const float* v_new, float* out, int32_t batch, int32_t n_q,
                                                  int32_t Hq, float alpha, int32_t causal, const int32_t* q_start,
                                                  const int32_t* block_table, int32_t max_pages, int32_t max_seq_len,
                                                  void* workspace, size_t ws_bytes, void* stream) {
  // the prefix lengths are q_start: they bound the packed tokens and the window read here
  kvq_status st = check_attend_args(c, q, batch, Hq, block_table, max_pages, q_start, max_seq_len);
  if (st != KVQ_OK) return st;
  if (!out || !k_new || !v_new) return fail(KVQ_ERR_INVALID_ARG, "out, k_new and v_new must be non-null");
  if (n_q < 1) return fail(KVQ_ERR_INVALID_ARG, "n_q must be >= 1");
  if (n_q > max_seq_len) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len must bound q_start + n_q");
  if (causal != 0 && causal != 1) return fail(KVQ_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (c->n_recent > 0 && batch > c->max_batch) return fail(KVQ_ERR_INVALID_ARG, "batch above the window rings' max_batch");
  if ((int64_t)batch * n_q * Hq > 0x7fffffff) return fail(KVQ_ERR_UNSUPPORTED, "batch * n_q * num_q_heads above 2^31 - 1");
  if ((int64_t)batch * n_q * c->num_kv_heads * 2 > (int64_t)INT32_MAX)
    return fail(KVQ_ERR_INVALID_ARG, "too many rows in one store");
  const size_t need = kvq_prefill_workspace_bytes(batch, n_q, Hq, c->head_dim, max_seq_len);
  if (!workspace || ws_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  // slices of the window and chunk rows, each of at least kRowSlice rows, and as many as bring
  // their blocks to about 4096.  With a possible prefix (max_seq_len > n_q) they are the last groups
  // of prefill_partial's grid, after the packed chunks; without one they are the whole work and run
  // in prefill_rows_f32, with 64-row blocks at a higher occupancy.
  const bool sep = max_seq_len <= n_q;
  const int rpb = sep ? 64 : prefill_rows_per_block(c->layout, c->head_dim);
  const int nf32 = min(c->n_recent, max_seq_len) + n_q;
  const int64_t row_blocks = ((int64_t)n_q * (Hq / c->num_kv_heads) + rpb - 1) / rpb * c->num_kv_heads * batch;
  const int64_t want = (4096 + row_blocks - 1) / row_blocks;
  int slice = (int)((nf32 + want - 1) / want);
  slice = max(kRowSlice, (slice + 15) / 16 * 16);
  const int nwin = (nf32 + slice - 1) / slice;
  // packed tokens of the longest prefix: q_start <= max_seq_len - n_q, less its window
  const int chunk = sep ? kPrefillChunk
                        : prefill_chunk(row_blocks, max(0, max_seq_len - n_q - c->n_recent), nwin, slice, true,
                                        prefill_blocks_per_cu(c->layout, c->head_dim));
  AttendArgs a = make_args(c, q, Hq, n_q, alpha, block_table, max_pages, q_start, max_seq_len, chunk, workspace);
  a.causal = causal;
  a.skip = 0;   // every packed token precedes the chunk: nothing to skip
  a.q_start = causal ? q_start : nullptr;
  const int nch = chunks_of(max_seq_len, chunk);
  a.slice = slice;
  a.nwin = nwin;
  a.nc1 = nch + nwin;
  a.nwg = sep ? 0 : nwin;
  a.ngroups = sep ? 0 : nch + nwin;
  const int64_t gx = sep ? 0 : row_blocks * a.ngroups;
  const int64_t gw = sep ? row_blocks * nwin : 0;
  if (gx > 0x7fffffff || gw > 0x7fffffff) return fail(KVQ_ERR_UNSUPPORTED, "prefill grid above 2^31 - 1 blocks");
  const int rows = batch * n_q * Hq;
  const RowPrep w = prefill_ws((size_t)rows, c->head_dim, a.nc1);
  hipStream_t s = (hipStream_t)stream;
  unsigned char* wsb = (unsigned char*)workspace;
  if (c->layout == HAD) {   // the chunk's rows in the rotated basis, as the window keeps its rows
    a.kchunk = (const float*)(wsb + w.kc);
    a.vchunk = (const float*)(wsb + w.vc);
    if ((st = launch_rotate_rows(c, k_new, v_new, batch * n_q, (float*)(wsb + w.kc), (float*)(wsb + w.vc), s)) != KVQ_OK)
      return st;
  } else {
    a.kchunk = k_new;
    a.vchunk = v_new;
  }
  if ((st = launch_prepare_rows(c, q, rows, wsb, w, a, s)) != KVQ_OK) return st;
  if (gx > 0) {
    pick_prefill(c->layout, c->head_dim)(a, dim3((unsigned)gx), false, s);
    if ((st = check_launch("prefill partial kernel")) != KVQ_OK) return st;
  }
  if (gw > 0) {
    pick_prefill(c->layout, c->head_dim)(a, dim3((unsigned)gw), true, s);
    if ((st = check_launch("prefill f32-row kernel")) != KVQ_OK) return st;
  }
  // the store follows the attention on the stream: it rewrites window slots the prefix was read from
  if ((st = kvq_store_chunk(c, k_new, v_new, batch, n_q, q_start, block_table, max_pages, max_seq_len, stream)) != KVQ_OK)
    return st;
  return launch_reduce(c, out, batch, n_q * Hq, q_start, a.nc1, chunk, (const float*)workspace, s, a.nwin,
                       a.slice, causal ? n_q : 0, RunSplit{}, true);
}
