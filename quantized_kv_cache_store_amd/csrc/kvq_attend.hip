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

// A operand of the int8 Q K^T MFMA: codes 32 g + 8 r .. 32 g + 8 r + 7 of staged K row t (even
// elements in the low dword, odd in the high one, the order the query operand follows; the 8-bit
// layout's stored bytes as they are, in element order).
template <int L, class ST>
__device__ __forceinline__ long k_operand(const unsigned char* buf, int t, int g, int r) {
  constexpr int BIAS = CodeBias<L>::value;
  if (L == Q80) return *reinterpret_cast<const long*>(buf + ST::kbytes8(t, g, r));
  uint32_t lo, hi;
  if (L == Q60) {
    const unsigned char* krow = buf + ST::KP + t * ST::RS;
    const uint32_t x = *reinterpret_cast<const uint32_t*>(krow + 24 * g + 4 * r);
    const uint32_t t2 = *reinterpret_cast<const uint16_t*>(krow + 24 * g + 16 + 2 * r);
    q6_octet(x, t2, lo, hi);
  } else {
    uint32_t x = *reinterpret_cast<const uint32_t*>(buf + ST::kword(t, g, r));
    if (BIAS) x ^= 0x88888888u;
    lo = x & 0x0F0F0F0Fu;
    hi = (x >> 4) & 0x0F0F0F0Fu;
  }
  return __builtin_bit_cast(long, u32x2{lo, hi});
}

// One lane's V source for the P V MFMA: octet oc (elements 8 oc .. 8 oc + 7) of the step's tokens
// in the lane's eight k-slots (slot k: token 16 (k >> 2) + 4 r + (k & 3)), as biased codes, with
// the scale (and zero) pairs of consecutive slots.  Rows at or past t_end may hold anything, so
// their scales are zeroed.  Codes as bytes: q6_0 even elements in ev, odd in od; q8_0 elements
// 0..3 in ev, 4..7 in od; the 4-bit layouts the octet's nibbles in ev.
template <int L>
struct VOctet {
  uint32_t ev[8], od[8];
  h2 s2[4], z2[4];
};

template <int L, class ST, bool FULL>
__device__ __forceinline__ void load_voctet(const unsigned char* buf, int T0, int t_end, int oc, int r, VOctet<L>& v) {
  constexpr int SB = ST::SB;
  constexpr int BIAS = CodeBias<L>::value;
  const int grp = oc >> 2;           // its 32-element block
  uint32_t sz[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int tl = 16 * (k >> 2) + 4 * r + (k & 3);
    if (L == Q60) {
      const unsigned char* vrow = buf + ST::VP + tl * ST::RS;
      const uint32_t x = *reinterpret_cast<const uint32_t*>(vrow + 24 * grp + 4 * (oc & 3));
      const uint32_t t2 = *reinterpret_cast<const uint16_t*>(vrow + 24 * grp + 16 + 2 * (oc & 3));
      q6_octet(x, t2, v.ev[k], v.od[k]);
    } else if (L == Q80) {
      const uint2 x = *reinterpret_cast<const uint2*>(buf + ST::vbytes8(tl, oc));
      v.ev[k] = x.x ^ 0x80808080u;
      v.od[k] = x.y ^ 0x80808080u;
    } else {
      uint32_t x = *reinterpret_cast<const uint32_t*>(buf + ST::vword(tl, oc));
      if (BIAS) x ^= 0x88888888u;
      v.ev[k] = x;
      v.od[k] = 0;
    }
    const bool ok = FULL || T0 + tl < t_end;
    const unsigned char* vrec = buf + ST::VR + tl * SB;
    uint32_t w;
    if (L == ASYM) w = reinterpret_cast<const uint32_t*>(vrec)[grp];
    else if (L != HAD) w = (uint32_t)reinterpret_cast<const uint16_t*>(vrec)[grp];
    else w = 0u;
    sz[k] = ok ? w : 0u;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v.s2[i] = as_h2(__builtin_amdgcn_perm(sz[2 * i + 1], sz[2 * i], 0x05040100u));
    v.z2[i] = as_h2(__builtin_amdgcn_perm(sz[2 * i + 1], sz[2 * i], 0x07060302u));
  }
}

// A operand of the f16 P V MFMA for element e of the octet: V^T[8 oc + e][slot k] as fp16,
// dequantised ((code | 0x6400) is 1024 + code in fp16, then scale and zero).
template <int L>
__device__ __forceinline__ v8h v_operand(const VOctet<L>& v, int e, uint32_t magic) {
  constexpr int BIAS = CodeBias<L>::value;
  v8h A;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t bsel = (uint32_t)(L == Q80 ? (e & 3) : (e >> 1));
    const uint32_t sel = bsel | (0x0Cu << 8) | ((4u + bsel) << 16) | (0x0Cu << 24);
    uint32_t pair;
    if (L == Q60 || L == Q80) {
      const bool hi = L == Q80 ? (e >> 2) != 0 : (e & 1) != 0;
      const uint32_t src_a = hi ? v.od[2 * i] : v.ev[2 * i];
      const uint32_t src_b = hi ? v.od[2 * i + 1] : v.ev[2 * i + 1];
      pair = __builtin_amdgcn_perm(src_b, src_a, sel) | magic;
    } else {
      const uint32_t y = __builtin_amdgcn_perm(v.ev[2 * i + 1], v.ev[2 * i], sel);
      pair = (((e & 1) ? (y >> 4) : y) & 0x000F000Fu) | magic;
    }
    h2 x = as_h2(pair) - h2{(_Float16)(1024 + BIAS), (_Float16)(1024 + BIAS)};
    if (L == ASYM) x = x * v.s2[i] + v.z2[i];
    else if (L != HAD) x = x * v.s2[i];
    A[2 * i] = x[0];
    A[2 * i + 1] = x[1];
  }
  return A;
}

// Float-query mode: the scores (before the softmax scale) of the lane's four tokens t0 + j of one
// 16-token half, with the query in three int8 terms (prepare_row_lanes): per 32-element block, three
// int8 MFMAs on the same unpacked codes, folded at once into (254 I(q8) + I(r1)) * 254 + I(r2) (the
// bracket exact in i32) and, for the block layouts, times the block's scale (the offset term is added
// by the caller); the Hadamard layout sums the three terms over the whole row first and subtracts
// their offsets qoff[0..2].  Each block's three accumulators die with the block.
// One16: the 16-row tile's half (A = the half's tokens, B = qB as it is); else the 8-row tile, whose
// two halves share the MFMA tile (A = half h's tokens, B = the query in the columns of half h, the lane
// reading half hh).
template <int L, int D, class ST>
__device__ __forceinline__ void fq_scores(const unsigned char* kbuf, int arow, int t0, int r, bool one16,
                                          const long* qB, const long* qBl, const int* qoff, float* xq, int hh = 0) {
  constexpr int NG = D / 32;
  constexpr int SB = ST::SB;
  const int nh = one16 ? 1 : 2;
  if (L == HAD) {
    v4i a0 = v4i{0, 0, 0, 0}, a1 = v4i{0, 0, 0, 0}, a2 = v4i{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h >= nh) break;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const long A = k_operand<L, ST>(kbuf, one16 ? arow : 16 * h + arow, g, r);
        const bool on = one16 || hh == h;
        a0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, on ? qB[g] : 0, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, on ? qBl[g] : 0, a1, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, on ? qBl[NG + g] : 0, a2, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xq[j] = fmaf((float)(254 * (a0[j] - qoff[0]) + (a1[j] - qoff[1])), 254.0f, (float)(a2[j] - qoff[2]));
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) xq[j] = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    v4i a0 = v4i{0, 0, 0, 0}, a1 = v4i{0, 0, 0, 0}, a2 = v4i{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h >= nh) break;
      const long A = k_operand<L, ST>(kbuf, one16 ? arow : 16 * h + arow, g, r);
      const bool on = one16 || hh == h;
      a0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, on ? qB[g] : 0, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, on ? qBl[g] : 0, a1, 0, 0, 0);
      a2 = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, on ? qBl[NG + g] : 0, a2, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned char* rec = kbuf + ST::KR + (t0 + j) * SB;
      const uint32_t w = rec_word(rec, (L == ASYM) ? g : (g >> 1));
      const float sc = (float)as_h2(w)[(L == ASYM) ? 0 : (g & 1)];
      xq[j] = fmaf(sc, fmaf((float)(254 * a0[j] + a1[j]), 254.0f, (float)a2[j]), xq[j]);
    }
  }
}

// One 32-token step of a wave: Q K^T, online softmax, P V, all from the staged rows in `buf`.
// FULL: every token of the step is inside the chunk and visible to every row (no masking).
// Otherwise tokens at or past t_end are dropped (their staged rows may hold anything, so their
// scales are zeroed too) and tokens past `lim`, the limit of this lane's row, get p = 0.
// drow: flat row index of this lane's row for the score export (DBG), or -1.
// FQ: float-query mode; qBl holds the query's two residual terms r1 (blocks 0 .. NG - 1) and r2
// (NG .. 2 NG - 1), and every block dot becomes (254 I(q8) + I(r1)) * 254 + I(r2) (qsB and sqc come
// scaled to match; the Hadamard layout's qoff holds the three terms' offsets).
template <int L, int D, class ST, bool DBG, bool FULL, bool FQ>
__device__ __forceinline__ void attend_step(const AttendArgs& a, const unsigned char* buf, int T0, int t_end,
                                            int lim, long drow, int col, int r, const long* qB, const long* qBl,
                                            const float* qsB, const int* qoff, float sqc, uint32_t magic,
                                            float& m_run, float& l_run, int& e_run, v4f* oacc) {
  using T = Layout<L, D>;
  constexpr int NG = T::NG;
  constexpr int SG = T::SG;
  constexpr int SB = T::SB;
  constexpr int NO = D / 128;

  // ---------------- Q K^T on the int8 MFMA, scores of this lane's 8 tokens
  float xs[8];
  float vs_had[8];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    v4i acc[SG];
    float xq[4];   // float-query mode: the tokens' scores before the softmax scale
    if constexpr (FQ) {
      fq_scores<L, D, ST>(buf, 16 * tau + col, 16 * tau + 4 * r, r, true, qB, qBl, qoff, xq);
    } else {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const long A = k_operand<L, ST>(buf, 16 * tau + col, g, r);
        const long B = qB[g];
        if (L == HAD)
          acc[0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, g == 0 ? v4i{0, 0, 0, 0} : acc[0], 0, 0, 0);
        else
          acc[g] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, v4i{0, 0, 0, 0}, 0, 0, 0);
      }
    }
    // offset term: A[t = col][k = r] from the record of token 16*tau + col
    v4f xo = v4f{0.f, 0.f, 0.f, 0.f};
    if (L != HAD && L != Q80) {
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
        const int I = FQ ? 0 : acc[0][j] - qoff[0];
        x = *reinterpret_cast<const float*>(rec) * (FQ ? xq[j] : (float)I);
        if (DBG && ok && drow >= 0) a.dbg[(size_t)drow * a.max_seq_len + T0 + tl] = I;
        const float vsc = *reinterpret_cast<const float*>(buf + ST::VR + tl * SB);
        vs_had[tau * 4 + j] = ok ? vsc : 0.0f;
      } else {
        x = FQ ? xo[j] + xq[j] : xo[j];
#pragma unroll
        for (int g = 0; g < (FQ ? 0 : SG); ++g) {
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
  const float m_new = fmax_nc(m_run, smax);
  const float m_use = m_new == -INFINITY ? 0.0f : m_new;
  // Hadamard layout: the exponent of the largest V scale so far (a lane's 8 tokens, then the four
  // lane rows: all 32 tokens of the step)
  int e_new = e_run;
  if (L == HAD) {
    float vmax = vs_had[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) vmax = fmax_pos(vmax, vs_had[i]);   // scales >= 0
    e_new = max(e_run, vscale_exp(max_over_rows(vmax)));
  }
  // rescale the running sums only when some lane's maximum (or the V exponent) moved (rare after the
  // first steps)
  if (__any(m_new > m_run || e_new > e_run)) {
    const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
    l_run *= corr;
    const float ocorr = L == HAD ? __builtin_amdgcn_ldexpf(corr, e_run - e_new) : corr;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[i] *= ocorr;
  }
  m_run = m_new;
  e_run = e_new;
  float psum = 0.0f;
  v8h pB;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = __builtin_amdgcn_exp2f(xs[i] - m_use);
    psum += p;
    pB[i] = (_Float16)(L == HAD ? p * __builtin_amdgcn_ldexpf(vs_had[i], -e_new) : p);
  }
  l_run += psum;

  // ---------------- P V on the f16 MFMA, V^T built from the staged rows
#pragma unroll
  for (int o = 0; o < NO; ++o) {
    VOctet<L> v;
    load_voctet<L, ST, FULL>(buf, T0, t_end, col + 16 * o, r, v);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      oacc[o * 8 + e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v_operand<L>(v, e, magic), pB, oacc[o * 8 + e], 0, 0, 0);
  }
}

// Lane l and lane l ^ 8 of each 16-lane row exchange a value (DPP row rotation by 8).
__device__ __forceinline__ uint32_t half_swap_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
}
__device__ __forceinline__ float half_swap(float v) { return __builtin_bit_cast(float, half_swap_u(__builtin_bit_cast(uint32_t, v))); }

// The same step for a tile of at most 8 rows, which leaves half of a 16 x 16 MFMA tile idle in
// attend_step.  Here both 16-token halves of the step share one output tile: column n of the
// Q K^T tile is row n & 7 against the tokens of half n >> 3, obtained by running the int8 MFMA
// over the two halves with B operands that hold the rows' queries in their own half of the
// columns and zeros in the other.  Lane (col, r) so holds the scores of row col & 7
// for tokens 16 (col >> 3) + 4 r + j.  P V likewise covers 32 output elements per tile: column n
// accumulates element 8 m + 2 pt + (n >> 3) of row n & 7 (tile pt), with the numerators of lane
// n's row in the B operand of its own half and zeros in the other.  Integer scores, the softmax
// numerators and the accumulated products are the same as in attend_step (the idle half adds
// exact zeros); only the row sum l is added up in another order.
// `mid` runs between the K side (Q K^T, scores) and the V side (softmax, P V): the direct-load
// ring refills the K half of the slot there and waits for the V half.  `vdone` runs as soon as
// every read of the V half is done (the codes and scales held in registers), before the softmax and
// the P V work on them: the ring refills the V half there.
template <int L, int D, class ST, bool DBG, bool FULL, bool FQ, class MID, class VDONE>
__device__ __forceinline__ void attend_step8(const AttendArgs& a, const unsigned char* kbuf, const unsigned char* vbuf,
                                             int T0, int t_end,
                                             int lim, long drow, int col, int r, const long* qB, const long* qBl,
                                             const float* qsB, const int* qoff, float sqc,
                                             uint32_t magic, float& m_run, float& l_run, int& e_run, v4f* oacc,
                                             MID&& mid, VDONE&& vdone) {
  using T = Layout<L, D>;
  constexpr int NG = T::NG;
  constexpr int SG = T::SG;
  constexpr int SB = T::SB;
  constexpr int NO = D / 128;
  const int hh = col >> 3;

  // ---------------- Q K^T: both halves into one tile
  constexpr int NACC = SG == 1 ? 2 : SG;
  v4i acc[NACC];
  float xq[4];   // float-query mode: the tokens' scores before the softmax scale
  if constexpr (FQ) {
    fq_scores<L, D, ST>(kbuf, col, 16 * hh + 4 * r, r, false, qB, qBl, qoff, xq, hh);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const long A = k_operand<L, ST>(kbuf, 16 * h + col, g, r);
        const long B = (hh == h) ? qB[g] : 0;   // the rows' queries in the columns of half h
        if (L == HAD)
          acc[h] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, g == 0 ? v4i{0, 0, 0, 0} : acc[h], 0, 0, 0);
        else
          acc[g] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, h == 0 ? v4i{0, 0, 0, 0} : acc[g], 0, 0, 0);
      }
    }
  }
  v4f xo = v4f{0.f, 0.f, 0.f, 0.f};
  if (L != HAD && L != Q80) {   // the 8-bit K codes carry no offset
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const unsigned char* orec = kbuf + ST::KR + (16 * h + col) * SB;
#pragma unroll
      for (int i = 0; i < NG / 4; ++i) {
        const float av = (L == ASYM) ? rec_f16(orec, 2 * (4 * i + r) + 1) : rec_f16(orec, 4 * i + r);
        xo = __builtin_amdgcn_mfma_f32_16x16x4f32(av, (hh == h) ? qsB[i] : 0.0f, xo, 0, 0, 0);
      }
    }
  }
  float xs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tl = 16 * hh + 4 * r + j;
    const bool ok = FULL || T0 + tl < t_end;
    const bool vis = FULL || (ok && T0 + tl <= lim);
    const unsigned char* rec = kbuf + ST::KR + tl * SB;
    float x;
    if (L == HAD) {
      const int I = FQ ? 0 : acc[0][j] + acc[1][j] - qoff[0];
      x = *reinterpret_cast<const float*>(rec) * (FQ ? xq[j] : (float)I);
      if (DBG && ok && drow >= 0) a.dbg[(size_t)drow * a.max_seq_len + T0 + tl] = I;
    } else {
      x = FQ ? xo[j] + xq[j] : xo[j];
#pragma unroll
      for (int g = 0; g < (FQ ? 0 : SG); ++g) {
        const uint32_t w = rec_word(rec, (L == ASYM) ? g : (g >> 1));
        const float s = (float)as_h2(w)[(L == ASYM) ? 0 : (g & 1)];
        x = fmaf(s, (float)acc[g][j], x);
        if (DBG && ok && drow >= 0)
          a.dbg[((size_t)drow * a.max_seq_len + T0 + tl) * SG + g] = acc[g][j] - qoff[g];
      }
    }
    xs[j] = vis ? x * sqc : -INFINITY;
  }
  mid();
  if (DBG) {   // the score export: the V half is not read, but the ring's load counts expect its refill
    vdone();
    return;
  }

  // ---------------- the V half into registers: per octet group the codes and scale (zero) pairs of
  // the lane's 8 tokens; the Hadamard layout's per-token V scales of the lane's 4 tokens (zero past
  // the chunk's end).  Then the slot is free.
  VOctet<L> vo[NO];
#pragma unroll
  for (int o = 0; o < NO; ++o) load_voctet<L, ST, FULL>(vbuf, T0, t_end, col + 16 * o, r, vo[o]);
  float vsc[4];
  if (L == HAD) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = 16 * hh + 4 * r + j;
      const float v = *reinterpret_cast<const float*>(vbuf + ST::VR + tl * SB);
      vsc[j] = (FULL || T0 + tl < t_end) ? v : 0.0f;
    }
  }
  vdone();

  // ---------------- online softmax (base 2): a row's 32 scores sit in lanes (col, r), (col ^ 8, r)
  float smax = fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3]));
  smax = max_over_rows(smax);
  smax = fmax_nc(smax, half_swap(smax));
  const float m_new = fmax_nc(m_run, smax);
  const float m_use = m_new == -INFINITY ? 0.0f : m_new;
  // Hadamard layout: the exponent of the largest V scale so far (the four lane rows and the two
  // halves: all 32 tokens of the step)
  int e_new = e_run;
  if (L == HAD) {
    float vmax = max_over_rows(fmax_pos(fmax_pos(vsc[0], vsc[1]), fmax_pos(vsc[2], vsc[3])));   // scales >= 0
    vmax = fmax_nc(vmax, half_swap(vmax));
    e_new = max(e_run, vscale_exp(vmax));
  }
  if (__any(m_new > m_run || e_new > e_run)) {
    const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
    l_run *= corr;
    const float ocorr = L == HAD ? __builtin_amdgcn_ldexpf(corr, e_run - e_new) : corr;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] *= ocorr;
  }
  m_run = m_new;
  e_run = e_new;
  float psum = 0.0f;
  _Float16 ph[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float p = __builtin_amdgcn_exp2f(xs[j] - m_use);
    psum += p;
    ph[j] = (_Float16)(L == HAD ? p * __builtin_amdgcn_ldexpf(vsc[j], -e_new) : p);
  }
  l_run += psum;
  // B operand of P V: k-slots 0..3 hold half 0's tokens, 4..7 half 1's; the other half's
  // numerators of this row come from lane col ^ 8
  const uint32_t own0 = as_u32(h2{ph[0], ph[1]}), own1 = as_u32(h2{ph[2], ph[3]});
  const uint32_t oth0 = half_swap_u(own0), oth1 = half_swap_u(own1);
  // (pB0 lives in the columns of half 0, pB1 in those of half 1; each is zero in the other half)
  const v8h pB0 = __builtin_bit_cast(v8h, hh ? u32x4{0u, 0u, 0u, 0u} : u32x4{own0, own1, oth0, oth1});
  const v8h pB1 = __builtin_bit_cast(v8h, hh ? u32x4{oth0, oth1, own0, own1} : u32x4{0u, 0u, 0u, 0u});

  // ---------------- P V: tile pt of octet group o takes elements 2 pt (columns 0..7) and 2 pt + 1
#pragma unroll
  for (int o = 0; o < NO; ++o) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      oacc[o * 4 + pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v_operand<L>(vo[o], 2 * pt, magic), pB0, oacc[o * 4 + pt], 0, 0, 0);
      oacc[o * 4 + pt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v_operand<L>(vo[o], 2 * pt + 1, magic), pB1, oacc[o * 4 + pt], 0, 0, 0);
    }
  }
}

// The decode grid as a flat list of work items (a.rs.on): rows in order; in a row, its units (kv head,
// then row tile) in order; in a unit, its chunk groups at the run length run_span picks and then, with
// a window, the window's block.  The items take the first ids of the grid, which is sized for the
// shortest runs, so the ids past them exit at once after every item has been dispatched (empty blocks
// interleaved with the work cost 10-20 % in slot time and dispatch order on a uniform batch).
struct FlatBlock {
  int b, hk, tile, cg, span;
  bool window, valid;
};

__device__ inline FlatBlock flat_block(const AttendArgs& a, unsigned id, int tiles) {
  FlatBlock f{};
  auto len = [&](int bb) { return ((const_i32_ptr)a.seq_len)[bb]; };
  f.span = run_span(a.rs, a.n_recent, len);
  const unsigned k = (unsigned)(f.span / a.rs.half_chunk);   // 8, 4 or 3
  const unsigned um = (1u << a.rs.unit_shift) - 1u;
  const unsigned win = a.n_recent > 0 ? 1u : 0u;
  unsigned base = 0, local = 0, per_unit = 1;
  int found = -1;
  for (int b0 = 0; b0 < a.rs.batch; b0 += 16) {
    int S[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) S[j] = len(b0 + j < a.rs.batch ? b0 + j : a.rs.batch - 1);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int Sq = a.n_recent > 0 ? (S[j] > a.n_recent ? S[j] - a.n_recent : 0) : S[j];
      const unsigned q = ((unsigned)Sq + um) >> a.rs.unit_shift;
      const unsigned groups = k == 8u ? (q + 7u) >> 3 : (k == 4u ? (q + 3u) >> 2 : (q + 2u) / 3u);
      const unsigned n = b0 + j < a.rs.batch ? (groups + win) * (unsigned)a.rs.units : 0u;
      if (found < 0 && id < base + n) {
        found = b0 + j;
        local = id - base;
        per_unit = groups + win;
      }
      base += n;
    }
  }
  f.valid = found >= 0;
  if (!f.valid) return f;
  f.b = found;
  const unsigned unit = local / per_unit, c = local - unit * per_unit;
  f.hk = (int)(unit / (unsigned)tiles);
  f.tile = (int)(unit - (unsigned)f.hk * (unsigned)tiles);
  f.window = win != 0u && c == per_unit - 1u;
  f.cg = f.window ? 0 : (int)c;
  return f;
}

// Split-K partial kernel.  Block = four waves = four consecutive chunks of one (batch row,
// kv head, row tile); each wave streams its chunk in 32-token steps with NB - 1 steps of loads
// in flight and writes the chunk's partial per row (o unnormalised, m in base-2 logits, l).
// TR: rows per tile, 16 (attend_step) or 8 (attend_step8, for groups of at most 8 rows).
// Grid: x = row tile * ngroups + chunk group (the last group is the window when n_recent > 0),
// y = kv head, z = batch row.
template <int L, int D, int TR, bool FQ = false>
struct PartialShape {
  // 8-row tiles stream through LDS rings filled by direct loads, one of RK K slots and one of RV V
  // slots per wave; 16-row tiles through the register ring (NB slots: NB - 1 steps in flight while
  // one is consumed)
  static constexpr bool DMA = TR == 8;
  using ST = Step<L, D, DMA>;
  static constexpr int NB = (ST::SLOTS <= 5) ? 5 : (D == 128 ? 3 : 2);
  // Two K and two V slots, unless four slots per wave would leave LDS for less than two blocks per
  // CU (D = 256 rows of q6_0 and q8_0; those kernels' registers allow two blocks): then one V slot,
  // and one K slot as well where three slots are still too many.  A single slot is refilled as soon
  // as its step has read it, and the second block's waves cover the wait.
  static constexpr int HALF_BYTES = ST::HALF;
  static constexpr int RK = (TR == 8 && 4 * 3 * HALF_BYTES > 81920) ? 1 : 2;
  static constexpr int RV = (TR == 8 && 4 * 4 * HALF_BYTES > 81920) ? 1 : 2;
  static constexpr int RING = DMA ? 4 * (RK + RV) * ST::HALF : 4 * ST::BYTES;
  static constexpr int MERGE = 4 * TR * (D + 4) * 4;            // the four waves' chunk partials
  static constexpr int LDS = RING > MERGE ? RING : MERGE;       // per block
  // waves per SIMD: as many as four blocks' rings in 160 KiB of LDS allow, registers permitting (the
  // float-query mode's second and third query terms and accumulators need the registers of two: at three
  // its head_dim-128 kernels spilled 10-40 registers inside the loop and ran up to three times slower)
  static constexpr int LDS_WAVES = LDS <= 40960 ? 4 : (LDS <= 54613 ? 3 : 2);
  static constexpr int MIN_WAVES = DMA ? (FQ && LDS_WAVES > 2 ? 2 : LDS_WAVES) : 2;
};

template <int L, int D, bool DBG, int TR, bool FQ>
__global__ __launch_bounds__(256, (PartialShape<L, D, TR, FQ>::MIN_WAVES)) void attend_partial(AttendArgs a) {
  static_assert(!(DBG && FQ), "the score export has no float-query form");
  using T = Layout<L, D>;
  using PS = PartialShape<L, D, TR, FQ>;
  using ST = typename PS::ST;
  constexpr int NB = PS::NB;
  constexpr int NG = T::NG;
  constexpr int SG = T::SG;
  constexpr int NO = D / 128;
  constexpr int BIAS = CodeBias<L>::k_side;
  extern __shared__ __align__(16) unsigned char smem[];

  // Block numbering: chunk group fastest (measured faster than kv head or batch row fastest: blocks
  // that run together then stream neighbouring chunks of one (row, kv head)).  The chip runs block
  // id on XCD id % 8, and in a ragged batch only the low chunk groups of the short rows hold
  // tokens, so each (batch row, kv head, tile) rotates its chunk groups by its own index: their
  // first groups then spread over all XCDs instead of piling onto the same ones.
  // With a run length chosen from the rows' lengths (a.rs.on) the grid is a flat list instead (flat_block).
  const int nrows = a.n_q * a.G;
  int hk, b, tile, cg, span;
  bool window_block;
  if (!DBG && a.rs.on) {
    const FlatBlock f = flat_block(a, blockIdx.x, (nrows + TR - 1) / TR);
    if (!f.valid) return;
    hk = f.hk;
    b = f.b;
    tile = f.tile;
    cg = f.cg;
    span = f.span;
    window_block = f.window;
  } else {
    hk = blockIdx.y;
    b = blockIdx.z;
    tile = (int)blockIdx.x / a.ngroups;
    const int tiles = (int)gridDim.x / a.ngroups;
    const int rot = (int)((((long)b * gridDim.y + hk) * tiles + tile) % a.ngroups);
    cg = (int)blockIdx.x - tile * a.ngroups - rot;
    if (cg < 0) cg += a.ngroups;
    span = a.span;                               // tokens of each wave
    window_block = !DBG && a.n_recent > 0 && cg == a.ngroups - 1;
  }
  const int S = a.seq_len[b];
  const int Sq = a.n_recent > 0 ? max(0, S - a.n_recent) : S;   // quantised tokens
  const int row0 = TR * tile;
  const int nvalid = min(TR, nrows - row0);
  const int qs0 = a.causal ? a.q_start[b] : 0;
  if (window_block) {
    if (S > 0) window_tile_block<L, D>(a, smem, b, hk, S, row0, nvalid, qs0);
    return;
  }
  if (cg * 4 * span >= Sq) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t_begin = (cg * 4 + wave) * span;
  const int lim_min = row_limit(a, qs0, row0, nrows);               // first row of the tile
  const int lim_max = row_limit(a, qs0, row0 + nvalid - 1, nrows);  // last row: the tile's farthest limit
  int t_end = min(t_begin + span, Sq);
  if (a.skip && lim_max < t_end - 1) t_end = max(t_begin, lim_max + 1);   // causal skip
  const bool has_chunk = t_begin < Sq;          // the reduce reads this chunk's partial (wave-uniform)
  const bool active = t_begin < t_end;          // tokens to stream
  ChunkPages cp{};
  size_t row_first = 0;
  if constexpr (!PS::DMA) {
    cp = chunk_pages(a, b, t_begin, t_end, lane, active);
    row_first = active ? chunk_row(a, cp, hk, t_begin) : 0;
  }
  const int nsteps = active ? (t_end - t_begin + 31) / 32 : 0;

  // ---- prologue: this lane's row of the tile, prepared in the wave (int8 query in the B-operand
  // order, its scale and block sums; float-query mode: also the two residual terms, with the block
  // sums and the scale taken for (254 I(q8) + I(r1)) * 254 + I(r2)).  With 8-row tiles lane column
  // col serves row col & 7, and its operands are zero outside its half.  The row's elements and
  // the page entries of the ring's first steps are loaded together, then the ring's first steps
  // issued, so that the preparation's arithmetic runs while they are in flight.
  const int col = lane & 15;
  const int r = lane >> 4;
  const int rsel = TR == 8 ? (col & 7) : col;   // this lane's row within the tile
  const int hh = col >> 3;
  float qx[NG][8];
  load_row_lanes<D>(a.q + row_index(a, b, hk, row0 + min(rsel, nvalid - 1)) * D, r, qx);

  // LDS rings of RK K slots and RV V slots per wave (step s in K slot s % RK and V slot s % RV).
  // The K half of step s + RK is issued as soon as the K side of step s has read its slot, the
  // V half of step s + RV as soon as the V side has read its slot, so the issue order is K(j + RK),
  // V(j + RV) for j = ..., s - 1, s (the prologue issues the same order for negative j), and each
  // half is waited for only where it is first read.  Loads complete in issue order, so the count of
  // the groups issued after a half bounds the wait for it (stores in the loop, and the query row's
  // loads issued before the prologue's, only make such a wait longer).
  constexpr int RK = PS::RK, RV = PS::RV, MX = RK > RV ? RK : RV;
  constexpr int G = ST::GROUP, H = ST::HALF;
  static_assert(!PS::DMA || (2 * MX) * G <= 63, "load counter range");
  unsigned char* kring = smem + wave * (RK + RV) * H;
  unsigned char* vring = kring + RK * H;
  const uint32_t kr_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)kring);
  const uint32_t vr_lds = kr_lds + RK * H;
  auto rows = [&](int st) { return half_rows_s(a, b, hk, t_begin + 32 * st, t_end); };
  if constexpr (PS::DMA) {
    // The page runs of the ring's first steps are read (scalar loads) while the row's loads fly.
    // The row is then waited for before the ring's loads are issued: the compiler's own wait, at
    // the row's first use, counts only its loads and would also wait for every ring load issued
    // after them, so the preparation below would start only once the ring's first steps had
    // landed instead of running while they are in flight.
    HalfRows pro[MX];
#pragma unroll
    for (int k = 0; k < MX; ++k) pro[k] = k < nsteps ? rows(k) : HalfRows{0, 0};
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : : "v"(qx[g][i]));
#pragma unroll
    for (int j = -MX; j < 0; ++j) {
      const int k = j + RK, v = j + RV;
      if (k >= 0 && k < nsteps) issue_dma_half<ST, false>(a, pro[k], lane, kr_lds + k * H);
      if (v >= 0 && v < nsteps) issue_dma_half<ST, true>(a, pro[v], lane, vr_lds + v * H);
    }
  }
  long qB[NG];          // B operands (int8 query of the tile's rows), one aligned register pair each
  long qBl[2 * NG];     // float-query mode: the residual terms' B operands (r1, then r2)
  float qsB[NG / 4];    // offset-term operand: zero point (asym) or -bias * scale times the block sums
  // bias * sum(q8): the Hadamard scores and the score export use it (float-query mode, Hadamard
  // layout: the offsets of q8, r1 and r2)
  int qoff[SG < 3 ? 3 : SG];
  float sqc = 0.0f;
  {
    RowQ<D> rq;
    prepare_row_lanes<L, D, FQ>(qx, r, rq);
    float qsf[NG];   // each block's sum as the offset term takes it
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      qB[g] = rq.qB[g];
      qBl[g] = FQ ? rq.qBl[g] : 0;
      qBl[NG + g] = FQ ? rq.qBl[NG + g] : 0;
      qsf[g] = FQ ? fmaf((float)(254 * rq.qsum[g] + rq.qsuml[g]), 254.0f, (float)rq.qsuml[NG + g]) : (float)rq.qsum[g];
    }
#pragma unroll
    for (int i = 0; i < NG / 4; ++i) {
      const float qs = r == 0 ? qsf[4 * i] : r == 1 ? qsf[4 * i + 1] : r == 2 ? qsf[4 * i + 2] : qsf[4 * i + 3];
      qsB[i] = (L == ASYM) ? qs : -(float)BIAS * qs;
    }
#pragma unroll
    for (int t = 0; t < (SG < 3 ? 3 : SG); ++t) {
      // term t of the Hadamard float-query mode, else block t
      const int* src = t == 0 || !FQ || L != HAD ? rq.qsum : rq.qsuml + (t - 1) * NG;
      int sum = 0;
      if (L == HAD) {
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) sum += src[gg];
      } else {
        sum = t < NG ? rq.qsum[t] : 0;
      }
      qoff[t] = BIAS * sum;
    }
    sqc = rq.sq * a.alpha * KVQ_LOG2E;
    if (FQ) sqc = sqc / 64516.0f;
  }
  const int lim = row_limit(a, qs0, row0 + rsel, nrows);
  const long drow = (DBG && rsel < nvalid) ? (long)row_index(a, b, hk, row0 + rsel) : -1;   // score export only
  if (DBG && !has_chunk) return;

  float m_run = -INFINITY, l_run = 0.0f;
  int e_run = kNoExp;   // Hadamard layout: the accumulators are in units of 2^e_run
  constexpr int NACC = TR == 8 ? D / 32 : D / 16;
  v4f oacc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) oacc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  uint32_t magic;   // fp16 "1024 + code" exponent bits, kept in a VGPR so v_and_or_b32 can take it
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  // The chunk's partial per row (o unnormalised, m, l) into the block's merge area in LDS, rows
  // of D + 4 floats per wave.
  auto write_partial_lds = [&](float* mo) {
    float l = sum_over_rows(l_run);
    if (TR == 8) l += half_swap(l);   // the row's other half of the tokens
    float* dst = mo + rsel * partial_stride(D);
    const float us = L == HAD ? __builtin_amdgcn_ldexpf(1.0f, e_run) : 1.0f;   // the accumulators' unit
    if (TR == 8) {
#pragma unroll
      for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[8 * (4 * r + j + 16 * o) + 2 * pt + hh] = oacc[o * 4 + pt][j] * us;
    } else {
#pragma unroll
      for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[8 * (4 * r + j + 16 * o) + e] = oacc[o * 8 + e][j] * us;
    }
    if (r == 0 && (TR == 16 || hh == 0)) {
      dst[D] = m_run;
      dst[D + 1] = l;
    }
  };

  auto step = [&](const unsigned char* kbuf, const unsigned char* vbuf, int T, auto&& mid, auto&& vdone) {
    const bool full = T + 32 <= t_end && T + 31 <= lim_min;
    if (TR == 8) {
      if (full)
        attend_step8<L, D, ST, DBG, true, FQ>(a, kbuf, vbuf, T, t_end, lim, drow, col, r, qB, qBl, qsB, qoff, sqc,
                                              magic, m_run, l_run, e_run, oacc, mid, vdone);
      else
        attend_step8<L, D, ST, DBG, false, FQ>(a, kbuf, vbuf, T, t_end, lim, drow, col, r, qB, qBl, qsB, qoff, sqc,
                                               magic, m_run, l_run, e_run, oacc, mid, vdone);
    } else {
      if (full)
        attend_step<L, D, ST, DBG, true, FQ>(a, kbuf, T, t_end, lim, drow, col, r, qB, qBl, qsB, qoff, sqc, magic,
                                             m_run, l_run, e_run, oacc);
      else
        attend_step<L, D, ST, DBG, false, FQ>(a, kbuf, T, t_end, lim, drow, col, r, qB, qBl, qsB, qoff, sqc, magic,
                                              m_run, l_run, e_run, oacc);
    }
  };

  if constexpr (PS::DMA) {
    auto wait_groups = [](int n) {
      switch (n) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<G>(); break;
        case 2: wait_vm<2 * G>(); break;
        case 3: wait_vm<3 * G>(); break;
        case 4: wait_vm<(4 * G <= 63 ? 4 * G : 63)>(); break;
        case 5: wait_vm<(5 * G <= 63 ? 5 * G : 63)>(); break;
        case 6: wait_vm<(6 * G <= 63 ? 6 * G : 63)>(); break;
        default: wait_vm<(7 * G <= 63 ? 7 * G : 63)>(); break;
      }
    };
    auto span_count = [](int lo, int hi) { return hi >= lo ? hi - lo + 1 : 0; };
    __builtin_amdgcn_s_setprio(3);   // lowered by progress in the loop below, after the steps
    // p2, p1, p0: the first s with 8 (s + 1) >= 4, 6, 7 nsteps (computed once: no division per step)
    const int p2 = (4 * nsteps + 7) / 8 - 1, p1 = (6 * nsteps + 7) / 8 - 1, p0 = (7 * nsteps + 7) / 8 - 1;
    // Steps s >= S0 with s + MX < nsteps are the steady part: no count below is clipped by the
    // chunk's ends, so the K wait counts 2 RK - 1 groups and the V wait 2 RV - 1.  Waits with these
    // constant counts skip the compare-and-branch ladder that wait_groups compiles to.
    constexpr int S0 = RK - RV > 0 ? RK - RV : (RV - 1 - RK > 0 ? RV - 1 - RK : 0);
    constexpr int NK = (2 * RK - 1) * G <= 63 ? (2 * RK - 1) * G : 63;   // a smaller count only waits longer
    constexpr int NV = (2 * RV - 1) * G <= 63 ? (2 * RV - 1) * G : 63;
    int ks = 0, vs = 0;   // slots of step s
    for (int s = 0; s < nsteps; ++s) {
      const bool k_next = s + RK < nsteps, v_next = s + RV < nsteps;
      const HalfRows hk_next = k_next ? rows(s + RK) : HalfRows{0, 0};
      const HalfRows hv_next = v_next ? rows(s + RV) : HalfRows{0, 0};
      // K of step s: then K(s + 1 .. s + RK - 1) and V(s - RK + RV .. s + RV - 1)
      const bool steady = s + MX < nsteps && s >= S0;
      if (steady)
        wait_vm<NK>();
      else
        wait_groups(span_count(s + 1, min(nsteps - 1, s + RK - 1)) +
                    span_count(max(0, s - RK + RV), min(nsteps - 1, s + RV - 1)));
      step(kring + ks * H, vring + vs * H, t_begin + 32 * s, [&]() {
        if (k_next) issue_dma_half<ST, false>(a, hk_next, lane, kr_lds + ks * H);
        // V of step s: then K(s - RV + 1 + RK .. s + RK) and V(s + 1 .. s + RV - 1)
        if (steady)
          wait_vm<NV>();
        else
          wait_groups(span_count(max(0, s - RV + 1 + RK), min(nsteps - 1, s + RK)) +
                      span_count(s + 1, min(nsteps - 1, s + RV - 1)));
      }, [&]() {
        if (v_next) issue_dma_half<ST, true>(a, hv_next, lane, vr_lds + vs * H);
      });
      ks = ks + 1 == RK ? 0 : ks + 1;
      vs = vs + 1 == RV ? 0 : vs + 1;
      // Issue priority by progress: a SIMD's waves (one from each of up to four blocks, equal work) are
      // otherwise served oldest first, so they finished one after another and the launch ended on a
      // SIMD holding a single wave (batch 8: live waves fell by quarters from 120 us of a 235 us
      // launch).  Each wave starts at 3 and drops to 2, 1 and 0 at 1/2, 3/4 and 7/8 of its run, so
      // waves ahead yield to waves behind and all finish within about 30 us (measured 236-243 ->
      // 224-230 us for that launch).
      if (s == p2) __builtin_amdgcn_s_setprio(2);
      if (s == p1) __builtin_amdgcn_s_setprio(1);
      if (s == p0) __builtin_amdgcn_s_setprio(0);
    }
  } else {
    unsigned char* buf = smem + wave * ST::BYTES;
    u32x4 pre[NB][ST::SLOTS];
    // Software pipeline over a ring of NB register slots, all loads issued inside the loop (nothing
    // is in flight at entry, so the compiler's load-counter waits stay exact): iteration i issues
    // step i into slot i % NB and consumes step i - (NB - 1) from slot (i + 1) % NB.  Issues past
    // the last step read a few bytes of the chunk's first rows (cache hits) so every iteration
    // issues the same loads.
    const int kend = nsteps > 0 ? nsteps + NB - 1 : 0;
    for (int k0 = 0; k0 < kend; k0 += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int si = k0 + k;
        const int Ti = t_begin + 32 * si;
        issue_step<L, D>(a, half_rows(a, cp, hk, Ti, t_end, row_first), lane, pre[k], si >= nsteps);
        const int su = si - (NB - 1);
        if (su >= 0 && su < nsteps) {
          stage_step<L, D>(buf, lane, pre[(k + 1) % NB]);
          step(buf, buf, t_begin + 32 * su, [] {}, [] {});
        }
      }
    }
  }
  if (DBG) return;

  // ---------------- merge of the block's four chunk partials (the first level of the online-softmax
  // merge, in a fixed order), written as the partial of the chunk group cg
  float* merge = reinterpret_cast<float*>(smem);
  __syncthreads();                                  // every wave is done with its ring
  write_partial_lds(merge + wave * TR * partial_stride(D));
  __syncthreads();
  {
    constexpr int TPR = 256 / TR;                   // threads per row
    constexpr int EPT = D / TPR;                    // elements per thread
    const int tid = threadIdx.x;
    const int row = tid / TPR, e0 = (tid % TPR) * EPT;
    if (row < nvalid) {
      const float* src = merge + row * partial_stride(D);
      constexpr int WS = TR * partial_stride(D);    // one wave's area
      float mk[4], M = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mk[k] = src[k * WS + D];
        M = fmaxf(M, mk[k]);
      }
      float w[4], l = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[k] = mk[k] == -INFINITY ? 0.0f : exp2f(mk[k] - M);
        l += w[k] * src[k * WS + D + 1];
      }
      float* dst = a.ws + (row_index(a, b, hk, row0 + row) * a.nc1 + cg) * partial_stride(D);
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        float o = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) o += w[k] * src[k * WS + e0 + e];
        dst[e0 + e] = o;
      }
      if (tid % TPR == 0) {
        dst[D] = M;
        dst[D + 1] = l;
      }
    }
  }
}

// Online-softmax merge of the chunk partials of each row (flat index (b * n_q + i) * Hq + h);
// Hadamard layout: rotate back.  W waves per row (4 / W rows per block): the row's waves split
// its chunks and, when W > 1, combine through LDS in a fixed order (deterministic).  Lane l owns
// output elements l * E .. l * E + E - 1; the rotation runs in registers, butterflies inside a
// lane for strides below E and between lanes above, in the stage order of the encoding
// (h = 1, 2, ..., D / 2, then 1 / sqrt(D)).
// nwin_always > 0: the last nwin_always slots hold partials of every row (full-precision prefill:
// the slices of its f32 rows), whatever the window; else the last slot holds the window's partial
// when there is a window and the row is not empty.  NARROW: the prefill's records (narrow_stride:
// f16 numerators and an exponent), else the decode's f32 ones.
template <int D, bool ROT, int W, bool NARROW>
__global__ __launch_bounds__(256) void attend_reduce(const float* ws, float* out, const int32_t* seq_len,
                                                     int rows_per_b, int nc1, int chunk, int n_recent,
                                                     long total_rows, int nwin_always, int slice, int causal_nq,
                                                     RunSplit rs) {
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
  const int PST = NARROW ? narrow_stride(D) : partial_stride(D);
  constexpr int MO = NARROW ? D / 2 : D;            // the record's m, l (and exponent) after the numerators
  const float* base = ws + (size_t)rr * nc1 * PST;
  // Narrow records with one wave per row and at most 64 slots: lane j loads slot j's (m, l, x) together
  // with the row length, and the numerators of every partial the row uses follow in one batch of up to
  // 16 loads, so a row costs about two dependent memory round trips instead of one per 4 partials.
  const bool fast = NARROW && W == 1 && nc1 <= 64;
  float rm = -INFINITY, rl = 0.0f;
  int rx = 0;
  if (fast && lane < nc1) {
    const float* rec = base + (size_t)lane * PST + MO;
    rm = rec[0];
    rl = rec[1];
    rx = reinterpret_cast<const int*>(rec)[2];
  }
  const int S = seq_len[b];
  const int Sq = n_recent > 0 ? max(0, S - n_recent) : S;
  if (rs.on) chunk = 4 * run_span(rs, n_recent, [&](int bb) { return ((const_i32_ptr)seq_len)[bb]; });
  const int nq = (Sq + chunk - 1) / chunk;
  int nw = nwin_always > 0 ? nwin_always : ((n_recent > 0 && S > 0) ? 1 : 0);
  if (nwin_always > 0 && causal_nq > 0) {   // the slices this query's causal limit reaches
    const int i = (int)(rr % rows_per_b) / (rows_per_b / causal_nq);
    nw = min(nw, (min(S, n_recent) + i) / slice + 1);
  }
  const int cnt = nq + nw;
  const int wbase = nc1 - (nwin_always > 0 ? nwin_always : 1) - nq;   // slot of partial i >= nq: wbase + i
  float o[E], l = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.0f;
  if (fast) {
    // slots in use: [0, nq) and [wbase + nq, wbase + cnt); the others may hold anything
    const bool used = lane < nq || (lane >= wbase + nq && lane < wbase + cnt);
    const float mj = used ? rm : -INFINITY;
    float M = mj;
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m));
    const float w = mj == -INFINITY ? 0.0f : exp2f(mj - M);
    float lw = mj == -INFINITY ? 0.0f : w * rl;
    for (int m = 1; m < 64; m <<= 1) lw += __shfl_xor(lw, m);
    l = lw;
    const int wx = __float_as_int(__builtin_amdgcn_ldexpf(w, rx));   // w * 2^x: the numerators' weight
    for (int i0 = 0; i0 < cnt; i0 += 16) {
      uint32_t hv[16][E / 2];
      float wk[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int i = i0 + k;
        if (i < cnt) {
          const int slot = i < nq ? i : wbase + i;
          const uint32_t* hw = reinterpret_cast<const uint32_t*>(base + (size_t)slot * PST) + lane * (E / 2);
          if constexpr (E == 2) {
            hv[k][0] = hw[0];
          } else {
            const u32x2 t = *reinterpret_cast<const u32x2*>(hw);
            hv[k][0] = t[0];
            hv[k][1] = t[1];
          }
          wk[k] = __int_as_float(__builtin_amdgcn_readlane(wx, slot));
        } else {
#pragma unroll
          for (int q = 0; q < E / 2; ++q) hv[k][q] = 0u;
          wk[k] = 0.0f;
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] += wk[k] * (float)as_h2(hv[k][e / 2])[e & 1];
    }
  } else {
    float M = -INFINITY;
    for (int i = sub * 64 + lane; i < cnt; i += 64 * W) M = fmaxf(M, base[(size_t)(i < nq ? i : wbase + i) * PST + MO]);
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m));
    if (W > 1) {
      if (lane == 0) red_m[wave] = M;
      __syncthreads();
      const int w0 = wave - sub;
      M = red_m[w0];
      for (int k = 1; k < W; ++k) M = fmaxf(M, red_m[w0 + k]);
    }
#pragma unroll 4
    for (int i = sub; i < cnt; i += W) {
      const float* p = base + (size_t)(i < nq ? i : wbase + i) * PST;
      const float mc = p[MO];
      const float w = (mc == -INFINITY) ? 0.0f : exp2f(mc - M);
      l += w * p[MO + 1];
      if constexpr (NARROW) {
        const float wx = __builtin_amdgcn_ldexpf(w, reinterpret_cast<const int*>(p)[MO + 2]);
        const uint32_t* hw = reinterpret_cast<const uint32_t*>(p) + lane * (E / 2);
        uint32_t hv[E / 2];
        if constexpr (E == 2) {
          hv[0] = hw[0];
        } else {
          const u32x2 t = *reinterpret_cast<const u32x2*>(hw);
          hv[0] = t[0];
          hv[1] = t[1];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] += wx * (float)as_h2(hv[e / 2])[e & 1];
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] += w * p[lane * E + e];
      }
    }
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

template <int L, int D, bool DBG, int TR, bool FQ>
static void launch_partial(const AttendArgs& a, dim3 grid, int n_recent, hipStream_t st) {
  size_t lds = PartialShape<L, D, TR, FQ>::LDS;
  if (n_recent > 0 && (size_t)window_lds_bytes<D>() > lds) lds = window_lds_bytes<D>();
  if (lds > 65536)
    (void)hipFuncSetAttribute((const void*)attend_partial<L, D, DBG, TR, FQ>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
  hipLaunchKernelGGL((attend_partial<L, D, DBG, TR, FQ>), grid, dim3(256), lds, st, a);
}

typedef void (*partial_fn)(const AttendArgs&, dim3, int, hipStream_t);

// Rows per tile of the decode kernel: 8 when a (batch row, kv head) has at most 8 query rows.
static inline int tile_rows(const AttendArgs& a) { return a.n_q * a.G <= 8 ? 8 : 16; }

template <bool DBG, bool FQ = false>
static partial_fn pick_partial(int layout, int D, int tr) {
  const int di = (D == 256 ? 1 : 0) + (tr == 8 ? 2 : 0);
#define KVQ_PARTIALS(L)                                                                                       \
  { launch_partial<L, 128, DBG, 16, FQ>, launch_partial<L, 256, DBG, 16, FQ>, launch_partial<L, 128, DBG, 8, FQ>, \
    launch_partial<L, 256, DBG, 8, FQ> }
  static const partial_fn tab[kNumLayouts][4] = {KVQ_PARTIALS(HAD), KVQ_PARTIALS(Q40), KVQ_PARTIALS(Q60),
                                                 KVQ_PARTIALS(ASYM), KVQ_PARTIALS(Q80)};
#undef KVQ_PARTIALS
  return tab[layout][di];
}

// Tokens per wave of the decode kernel, a function of the call's shape and the device (the partial
// and the reduce calls agree on it).  Every level of the split-K merge is the same online-softmax
// update, so a wave can take up to four consecutive chunks as one run, merged in its registers,
// while one round of resident waves (four per SIMD) still has work for all of them: the grid then
// needs fewer rounds of the chip, each of which ends with the blocks' barriers, merges and partial
// stores, during which their LDS and wave slots stream nothing (the register-ring kernel also
// needs the run's pages to fit its page registers).  With few waves the runs get shorter instead,
// down to a quarter chunk, while the doubled wave count still leaves half the wave slots free: a
// short context then spreads over more CUs (a wave's run is a serial chain of steps).  Halving the
// runs where that would fill every slot measured slower (batch 1 at 128K: 42 us against 39).  Every
// span keeps 4 * span >= chunk, so the partial slots fit the workspace.
static int decode_span(const kvq_cache* c, int batch, int Hq, int max_seq_len, int chunk) {
  const int G = Hq / c->num_kv_heads;
  const int tr = G <= 8 ? 8 : 16;
  const int64_t waves = (int64_t)batch * c->num_kv_heads * ((G + tr - 1) / tr) * chunks_of(max_seq_len, chunk);
  const int64_t resident = (int64_t)device_cus() * 16;
  int cpw = 1;
  while (cpw < 4 && waves >= resident * 2 * cpw && (2 * cpw * chunk) / c->page_size + 1 < 64 * kPageRegs) cpw *= 2;
  if (cpw > 1) return cpw * chunk;
  int span = chunk;
  for (int64_t w = waves; span > chunk / 4 && span % 64 == 0 && 4 * w <= resident; w *= 2) span /= 2;
  return span;
}

// Workspace of the decode: room for the partials [B x Hq x (chunks + 1) x (D + 4)] f32 (the decode
// kernel prepares its query rows itself).  A call writes fewer: one partial per group of a block's
// four wave runs (decode_span) and the window's, so its partial slots per row are
// decode_slots(...) <= chunks + 1, and decode_partials_bytes(...) is what it touches.
static size_t decode_ws_bytes(int batch, int Hq, int D, int max_seq_len, int chunk) {
  const size_t rows = (size_t)batch * Hq;
  const size_t nc1 = (size_t)chunks_of(max_seq_len, chunk) + 1;
  return rows * nc1 * partial_stride(D) * sizeof(float);
}

static int decode_slots(int max_seq_len, int span) { return chunks_of(max_seq_len, 4 * span) + 1; }

// Blocks of the decode partial kernel resident on one CU: a block holds one wave per SIMD, so the
// kernel's waves per SIMD (its launch bound, which its registers meet), or fewer where fewer blocks'
// LDS fits in 160 KiB.
template <int L, int D, int TR, bool FQ>
static int partial_blocks_per_cu(int n_recent) {
  size_t lds = PartialShape<L, D, TR, FQ>::LDS;
  if (n_recent > 0 && (size_t)window_lds_bytes<D>() > lds) lds = window_lds_bytes<D>();
  const int by_lds = (int)(163840 / lds);
  const int w = PartialShape<L, D, TR, FQ>::MIN_WAVES;
  return by_lds < w ? by_lds : w;
}

static int blocks_per_cu(int layout, int D, int tr, bool fq, int n_recent) {
  typedef int (*fn)(int);
  const int di = (D == 256 ? 1 : 0) + (tr == 8 ? 2 : 0) + (fq ? 4 : 0);
#define KVQ_RES(L)                                                                                               \
  { partial_blocks_per_cu<L, 128, 16, false>, partial_blocks_per_cu<L, 256, 16, false>,                        \
    partial_blocks_per_cu<L, 128, 8, false>, partial_blocks_per_cu<L, 256, 8, false>,                          \
    partial_blocks_per_cu<L, 128, 16, true>, partial_blocks_per_cu<L, 256, 16, true>,                          \
    partial_blocks_per_cu<L, 128, 8, true>, partial_blocks_per_cu<L, 256, 8, true> }
  static const fn tab[kNumLayouts][8] = {KVQ_RES(HAD), KVQ_RES(Q40), KVQ_RES(Q60), KVQ_RES(ASYM), KVQ_RES(Q80)};
#undef KVQ_RES
  return tab[layout][di](n_recent);
}

// The decode's split for a call: a fixed run length (decode_span), or, when even runs of four chunks
// leave more blocks than the chip holds at once (a batch of several rows), the run length chosen per
// call from the rows' lengths (run_span, on the device), with the grid and the partial slots sized for
// the shortest candidate, a chunk and a half.  The 16-row kernel keeps a run's page entries in registers, so
// that choice needs the longest candidate's pages to fit them.
struct DecodePlan {
  int span;      // the grid's run length
  int nc1;       // partial slots per row
  RunSplit rs;
};

static DecodePlan decode_plan(const kvq_cache* c, int batch, int Hq, int max_seq_len, int chunk, bool fq) {
  DecodePlan p{};
  p.span = decode_span(c, batch, Hq, max_seq_len, chunk);
  const int G = Hq / c->num_kv_heads;
  const int tr = G <= 8 ? 8 : 16;
  const int units = c->num_kv_heads * ((G + tr - 1) / tr);
  const long slots = (long)device_cus() * blocks_per_cu(c->layout, c->head_dim, tr, fq, c->n_recent);
  const long longest = (long)batch * units * chunks_of(max_seq_len, 16 * chunk);   // blocks of four-chunk runs
  const long most = (long)batch * units * chunks_of(max_seq_len, 6 * chunk);       // of the shortest candidate
  const bool pages_fit = tr == 8 || (4 * chunk) / c->page_size + 1 < 64 * kPageRegs;
  const bool pow2 = (chunk & (chunk - 1)) == 0;
  if (batch > 1 && batch <= 4096 && longest > slots && pages_fit && pow2 && slots > 0 && most < (1L << 31)) {
    p.rs = RunSplit{1, units, (int)slots, chunk / 2, __builtin_ctz((unsigned)(2 * chunk)), batch};
    p.span = kRunShortest * (chunk / 2);
  }
  p.nc1 = decode_slots(max_seq_len, p.span);
  return p;
}

size_t decode_partials_bytes(const kvq_cache* c, int batch, int Hq, int max_seq_len, int chunk) {
  const DecodePlan p = decode_plan(c, batch, Hq, max_seq_len, chunk, false);
  return (size_t)batch * Hq * p.nc1 * partial_stride(c->head_dim) * sizeof(float);
}

static kvq_status check_chunk(const kvq_cache* c, int32_t chunk) {
  if (chunk < 128 || chunk % 128) return fail(KVQ_ERR_INVALID_ARG, "chunk_tokens must be a positive multiple of 128");
  if ((chunk + c->page_size - 1) / c->page_size + 1 > 64 * kPageRegs)
    return fail(KVQ_ERR_UNSUPPORTED, "a chunk may span at most %d pages", 64 * kPageRegs - 1);
  return KVQ_OK;
}

template <int D, bool ROT, int W>
static void launch_reduce_w(float* out, long rows, int rows_per_b, const int32_t* seq_len, int nc1, int chunk,
                            int n_recent, const float* ws, hipStream_t s, int nwin_always, int slice, int causal_nq,
                            RunSplit rs, bool narrow) {
  const long blocks = (rows + (4 / W) - 1) / (4 / W);
  if (narrow)
    hipLaunchKernelGGL((attend_reduce<D, ROT, W, true>), dim3((unsigned)blocks), dim3(256), 0, s, ws, out, seq_len,
                       rows_per_b, nc1, chunk, n_recent, rows, nwin_always, slice, causal_nq, rs);
  else
    hipLaunchKernelGGL((attend_reduce<D, ROT, W, false>), dim3((unsigned)blocks), dim3(256), 0, s, ws, out, seq_len,
                       rows_per_b, nc1, chunk, n_recent, rows, nwin_always, slice, causal_nq, rs);
}

kvq_status launch_reduce(const kvq_cache* c, float* out, int32_t batch, int32_t rows_per_b, const int32_t* seq_len,
                         int nc1, int32_t chunk, const float* ws, hipStream_t s, int nwin_always, int slice,
                         int causal_nq, RunSplit rs, bool narrow) {
  const int wa = nwin_always;
  const long rows = (long)batch * rows_per_b;
  // one wave per row when there are rows enough to fill the chip, else four waves split each row
  const bool many = rows >= 4096;
  const bool rot = c->layout == HAD;
  const int n = c->n_recent;
  if (c->head_dim == 128) {
    if (rot) many ? launch_reduce_w<128, true, 1>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s, wa, slice, causal_nq, rs, narrow)
                  : launch_reduce_w<128, true, 4>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s, wa, slice, causal_nq, rs, narrow);
    else many ? launch_reduce_w<128, false, 1>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s, wa, slice, causal_nq, rs, narrow)
              : launch_reduce_w<128, false, 4>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s, wa, slice, causal_nq, rs, narrow);
  } else {
    if (rot) many ? launch_reduce_w<256, true, 1>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s, wa, slice, causal_nq, rs, narrow)
                  : launch_reduce_w<256, true, 4>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s, wa, slice, causal_nq, rs, narrow);
    else many ? launch_reduce_w<256, false, 1>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s, wa, slice, causal_nq, rs, narrow)
              : launch_reduce_w<256, false, 4>(out, rows, rows_per_b, seq_len, nc1, chunk, n, ws, s, wa, slice, causal_nq, rs, narrow);
  }
  return check_launch("attention reduce kernel");
}

}  // namespace kvq

using namespace kvq;

extern "C" size_t kvq_decode_workspace_bytes(int32_t batch, int32_t Hq, int32_t D, int32_t max_seq_len,
                                             int32_t chunk) {
  if (batch < 1 || Hq < 1 || (D != 128 && D != 256) || max_seq_len < 0 || chunk < 128 || chunk % 128) return 0;
  // +1 partial slot for the window (always reserved so the size does not depend on n_recent)
  return decode_ws_bytes(batch, Hq, D, max_seq_len, chunk);
}

// The split-K phase of decode, in the int8-query mode or (fq) the float-query mode, after the
// arguments were checked (decode_check) and with a workspace of at least decode_partials_bytes.
kvq_status kvq::decode_partial_ws(const kvq_cache* c, const float* q, int32_t batch, int32_t Hq, float alpha,
                                    const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                                    int32_t max_seq_len, int32_t chunk, void* workspace, void* stream, bool fq) {
  AttendArgs a = make_args(c, q, Hq, 1, alpha, block_table, max_pages, seq_len, max_seq_len, chunk, workspace);
  const int tr = tile_rows(a);
  const DecodePlan p = decode_plan(c, batch, Hq, max_seq_len, chunk, fq);
  a.span = p.span;
  a.rs = p.rs;
  a.ngroups = chunks_of(max_seq_len, 4 * a.span) + (c->n_recent > 0 ? 1 : 0);
  a.nc1 = p.nc1;   // the window's slot is the last
  const int64_t gx = grid_x(a, tr);
  if (gx == 0) return KVQ_OK;
  a.batch = batch;
  // the flat list (rs.on): every unit of every row, its chunk groups at the shortest runs and the window
  const dim3 grid = p.rs.on ? dim3((unsigned)((int64_t)batch * c->num_kv_heads * gx), 1, 1)
                            : dim3((unsigned)gx, c->num_kv_heads, batch);
  (fq ? pick_partial<false, true> : pick_partial<false, false>)(c->layout, c->head_dim, tr)(a, grid, c->n_recent,
                                                                                          (hipStream_t)stream);
  return check_launch("decode partial kernel");
}

// The reduce phase over the partials decode_partial_ws wrote for the same arguments: each partial
// slot holds a block's four wave runs of `span` tokens (merged by the partial kernel), the window's
// partial the last slot.
kvq_status kvq::decode_reduce_ws(const kvq_cache* c, float* out, int32_t batch, int32_t Hq, const int32_t* seq_len,
                                   int32_t max_seq_len, int32_t chunk, const void* workspace, void* stream, bool fq) {
  const DecodePlan p = decode_plan(c, batch, Hq, max_seq_len, chunk, fq);
  return launch_reduce(c, out, batch, Hq, seq_len, p.nc1, 4 * p.span, (const float*)workspace, (hipStream_t)stream, 0,
                       0, 0, p.rs);
}

static kvq_status check_decode_workspace(const kvq_cache* c, int32_t batch, int32_t Hq, int32_t max_seq_len,
                                         int32_t chunk, const void* workspace, size_t ws_bytes) {
  const size_t need = kvq_decode_workspace_bytes(batch, Hq, c->head_dim, max_seq_len, chunk);
  if (!workspace || ws_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  return KVQ_OK;
}

kvq_status kvq::decode_check(const kvq_cache* c, const float* q, int32_t batch, int32_t Hq,
                               const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                               int32_t max_seq_len, int32_t chunk) {
  kvq_status st = check_attend_args(c, q, batch, Hq, block_table, max_pages, seq_len, max_seq_len);
  if (st != KVQ_OK) return st;
  return check_chunk(c, chunk);
}

extern "C" kvq_status kvq_decode_split(const kvq_cache* c, int32_t batch, int32_t Hq, int32_t max_seq_len,
                                       int32_t chunk, int32_t* wave_tokens, int32_t* partial_tokens) {
  kvq_status st = validate_cache(c);
  if (st != KVQ_OK) return st;
  if (!wave_tokens || !partial_tokens) return fail(KVQ_ERR_INVALID_ARG, "wave_tokens and partial_tokens must be non-null");
  if (batch < 1 || Hq < 1 || Hq % c->num_kv_heads) return fail(KVQ_ERR_INVALID_ARG, "bad batch or num_q_heads");
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if ((st = check_chunk(c, chunk)) != KVQ_OK) return st;
  const DecodePlan p = decode_plan(c, batch, Hq, max_seq_len, chunk, false);
  const int span = p.rs.on ? run_span(p.rs, c->n_recent, [&](int) { return max_seq_len; }) : p.span;
  *wave_tokens = span;
  *partial_tokens = 4 * span;
  return KVQ_OK;
}

extern "C" kvq_status kvq_decode_split_lengths(const kvq_cache* c, int32_t batch, int32_t Hq,
                                               const int32_t* seq_len_host, int32_t max_seq_len, int32_t chunk,
                                               int32_t* wave_tokens, int32_t* partial_tokens) {
  kvq_status st = validate_cache(c);
  if (st != KVQ_OK) return st;
  if (!wave_tokens || !partial_tokens || !seq_len_host)
    return fail(KVQ_ERR_INVALID_ARG, "seq_len, wave_tokens and partial_tokens must be non-null");
  if (batch < 1 || Hq < 1 || Hq % c->num_kv_heads) return fail(KVQ_ERR_INVALID_ARG, "bad batch or num_q_heads");
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  for (int b = 0; b < batch; ++b)
    if (seq_len_host[b] < 0 || seq_len_host[b] > max_seq_len)
      return fail(KVQ_ERR_INVALID_ARG, "seq_len[%d] = %d outside [0, max_seq_len]", b, seq_len_host[b]);
  if ((st = check_chunk(c, chunk)) != KVQ_OK) return st;
  const DecodePlan p = decode_plan(c, batch, Hq, max_seq_len, chunk, false);
  const int span = p.rs.on ? run_span(p.rs, c->n_recent, [&](int b) { return seq_len_host[b]; }) : p.span;
  *wave_tokens = span;
  *partial_tokens = 4 * span;
  return KVQ_OK;
}

extern "C" kvq_status kvq_attend_decode_partial(const kvq_cache* c, const float* q, int32_t batch, int32_t Hq,
                                                float alpha, const int32_t* block_table, int32_t max_pages,
                                                const int32_t* seq_len, int32_t max_seq_len, int32_t chunk,
                                                void* workspace, size_t ws_bytes, void* stream) {
  kvq_status st = decode_check(c, q, batch, Hq, block_table, max_pages, seq_len, max_seq_len, chunk);
  if (st == KVQ_OK) st = check_decode_workspace(c, batch, Hq, max_seq_len, chunk, workspace, ws_bytes);
  if (st != KVQ_OK) return st;
  return decode_partial_ws(c, q, batch, Hq, alpha, block_table, max_pages, seq_len, max_seq_len, chunk, workspace,
                           stream, false);
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
  if ((st = check_decode_workspace(c, batch, Hq, max_seq_len, chunk, workspace, ws_bytes)) != KVQ_OK) return st;
  return decode_reduce_ws(c, out, batch, Hq, seq_len, max_seq_len, chunk, workspace, stream);
}

// Both phases, int8-query (fq = false) or float-query mode.
static kvq_status decode_both(const kvq_cache* c, const float* q, float* out, int32_t batch, int32_t Hq, float alpha,
                              const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                              int32_t max_seq_len, int32_t chunk, void* workspace, size_t ws_bytes, void* stream,
                              bool fq) {
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out must be non-null");
  kvq_status st = decode_check(c, q, batch, Hq, block_table, max_pages, seq_len, max_seq_len, chunk);
  if (st == KVQ_OK) st = check_decode_workspace(c, batch, Hq, max_seq_len, chunk, workspace, ws_bytes);
  if (st != KVQ_OK) return st;
  if ((st = decode_partial_ws(c, q, batch, Hq, alpha, block_table, max_pages, seq_len, max_seq_len, chunk, workspace,
                              stream, fq)) != KVQ_OK)
    return st;
  return decode_reduce_ws(c, out, batch, Hq, seq_len, max_seq_len, chunk, workspace, stream, fq);
}

extern "C" kvq_status kvq_attend_decode(const kvq_cache* c, const float* q, float* out, int32_t batch, int32_t Hq,
                                        float alpha, const int32_t* block_table, int32_t max_pages,
                                        const int32_t* seq_len, int32_t max_seq_len, int32_t chunk,
                                        void* workspace, size_t ws_bytes, void* stream) {
  return decode_both(c, q, out, batch, Hq, alpha, block_table, max_pages, seq_len, max_seq_len, chunk, workspace,
                     ws_bytes, stream, false);
}

extern "C" kvq_status kvq_attend_decode_float_q(const kvq_cache* c, const float* q, float* out, int32_t batch,
                                                int32_t Hq, float alpha, const int32_t* block_table,
                                                int32_t max_pages, const int32_t* seq_len, int32_t max_seq_len,
                                                int32_t chunk, void* workspace, size_t ws_bytes, void* stream) {
  return decode_both(c, q, out, batch, Hq, alpha, block_table, max_pages, seq_len, max_seq_len, chunk, workspace,
                     ws_bytes, stream, true);
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
  a.dbg = scores;
  a.kring = nullptr;
  a.vring = nullptr;
  a.ngroups = (chunks_of(max_seq_len, chunk) + 3) / 4;   // no window group: the export covers quantised tokens
  a.batch = batch;
  const int tr = tile_rows(a);
  const dim3 grid((unsigned)grid_x(a, tr), c->num_kv_heads, batch);
  pick_partial<true>(c->layout, c->head_dim, tr)(a, grid, 0, (hipStream_t)stream);
  return check_launch("score export kernel");
}
