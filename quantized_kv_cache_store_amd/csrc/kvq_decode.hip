// Fused compressed-domain decode attention: split-K partial kernel, f32 window
// partial, and the online-softmax reduce.
//
// [Open-TQ-Metal] Algorithm 1 (fused single pass over the packed cache, no
// dequantised S x d temporary) and the split-K paragraphs (chunks in parallel,
// each emitting o_c, m_c, l_c; a second phase merges them).  Scores are the
// integer dot int8(Q) . code(K) per 32-element block with the scales applied
// outside the reduction ([tract-RFC] Architecture > Data flow (decode)).
//
// gfx950 mapping.  One block of four waves handles one (batch row, kv head,
// chunk); each wave takes 32-token steps of the chunk.  For a step:
//   * Q K^T runs on v_mfma_i32_16x16x32_i8: A = 16 tokens x 32 codes of one
//     block (unpacked nibbles, one dword per lane), B = the int8 query of up to
//     16 heads of the kv head's GQA group (kept in registers for the block).
//     The i32 result per (token, head, block) is scaled by the block's scale.
//   * P V runs on v_mfma_f32_16x16x32_f16 with the output transposed,
//     C[d][head] += V^T[d][t] P^T[t][head]: the P^T operand is exactly the
//     softmax numerators the lane already holds from Q K^T (lane = head,
//     k-slots = its 8 tokens), so no shuffle is needed; the V^T operand is
//     built from the packed dwords of the same 8 tokens, nibble p of dword c
//     giving row d = 8c + p (fp16 "1024 + code" then an exact offset and the
//     block scale).
//   * the online softmax keeps m and l per head in the lanes that own the
//     head's column, so the rescale of the accumulators is lane-local.
// The four waves merge their (m, l, o) in LDS in a fixed order (deterministic).

#include "kvq_internal.h"

namespace kvq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

#define KVQ_LOG2E 1.4426950408889634f

struct DecodeArgs {
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
  int32_t* dbg;
  int Hkv, Hq, G, page_shift, n_recent, max_pages, chunk, nc1, max_seq_len;
  float alpha;
};

template <int D>
__host__ __device__ constexpr int prologue_lds_bytes() {
  return 16 * D * 4 + 16 * D + 16 * 4 + 16 * (D / 32) * 4;
}

__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// Physical row of logical token t of (batch b, kv head hk) in the planes.
__device__ __forceinline__ size_t plane_row(const DecodeArgs& a, int b, int hk, int t) {
  const int phys = a.block_table[(size_t)b * a.max_pages + (t >> a.page_shift)];
  return (((size_t)phys * a.Hkv + hk) << a.page_shift) + (size_t)(t & ((1 << a.page_shift) - 1));
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

// Window partial: exact f32 rows of the newest tokens (HAD: rotated basis).
template <int L, int D>
__device__ void window_partial(const DecodeArgs& a, unsigned char* smem, int b, int hk, int S) {
  float* qf = reinterpret_cast<float*>(smem);
  int8_t* q8 = reinterpret_cast<int8_t*>(qf + 16 * D);
  float* sq = reinterpret_cast<float*>(q8 + 16 * D);
  int* qsum = reinterpret_cast<int*>(sq + 16);
  float* sc = reinterpret_cast<float*>(smem + prologue_lds_bytes<D>());   // [G][W]
  const int tid = threadIdx.x;
  const int G = a.G;
  for (int idx = tid; idx < 16 * D; idx += 256) {
    const int row = idx / D;
    qf[idx] = row < G ? a.q[((size_t)b * a.Hq + hk * G + row) * D + idx % D] : 0.0f;
  }
  __syncthreads();
  prepare_query_lds<L, D>(qf, q8, sq, qsum);
  const int W = min(S, a.n_recent);
  const int w0 = S - W;
  const size_t ring0 = ((size_t)b * a.Hkv + hk) * a.n_recent;
  const float cl = a.alpha * KVQ_LOG2E;
  for (int idx = tid; idx < G * W; idx += 256) {
    const int h = idx / W, tt = idx % W;
    const float* kr = a.kring + (ring0 + (w0 + tt) % a.n_recent) * D;
    const float* qh = qf + h * D;
    float acc = 0.0f;
    for (int d = 0; d < D; d += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(kr + d);
      acc += qh[d] * k4.x + qh[d + 1] * k4.y + qh[d + 2] * k4.z + qh[d + 3] * k4.w;
    }
    sc[idx] = acc * cl;
  }
  __syncthreads();
  float* mrow = sc + 16 * W;
  float* lrow = mrow + 16;
  if (tid < G) {
    float m = -INFINITY;
    for (int tt = 0; tt < W; ++tt) m = fmaxf(m, sc[tid * W + tt]);
    float l = 0.0f;
    for (int tt = 0; tt < W; ++tt) {
      const float p = exp2f(sc[tid * W + tt] - m);
      sc[tid * W + tt] = p;
      l += p;
    }
    mrow[tid] = m;
    lrow[tid] = l;
  }
  __syncthreads();
  const int PST = partial_stride(D);
  for (int idx = tid; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    float o = 0.0f;
    for (int tt = 0; tt < W; ++tt) o += sc[h * W + tt] * a.vring[(ring0 + (w0 + tt) % a.n_recent) * D + d];
    float* dst = a.ws + (((size_t)b * a.Hq + hk * G + h) * a.nc1 + (a.nc1 - 1)) * PST;
    dst[d] = o;
    if (d == 0) {
      dst[D] = mrow[h];
      dst[D + 1] = lrow[h];
    }
  }
}

template <int L, int D, bool DBG>
__global__ __launch_bounds__(256) void decode_partial(DecodeArgs a) {
  using T = Layout<L, D>;
  constexpr int NG = T::NG;
  constexpr int SG = T::SG;
  constexpr int NO = D / 128;            // octets per lane: col and col + 16
  constexpr int BIAS = CodeBias<L>::value;
  extern __shared__ __align__(16) unsigned char smem[];

  const int c = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int S = a.seq_len[b];
  const int Sq = a.n_recent > 0 ? max(0, S - a.n_recent) : S;
  if (!DBG && a.n_recent > 0 && c == a.nc1 - 1) {
    if (S > 0) window_partial<L, D>(a, smem, b, hk, S);
    return;
  }
  const int t_begin = c * a.chunk;
  if (t_begin >= Sq) return;
  const int t_end = min(t_begin + a.chunk, Sq);
  const int G = a.G;

  // ---- prologue: query preparation for the GQA group of this kv head
  float* qf = reinterpret_cast<float*>(smem);
  int8_t* q8 = reinterpret_cast<int8_t*>(qf + 16 * D);
  float* sqv = reinterpret_cast<float*>(q8 + 16 * D);
  int* qsum = reinterpret_cast<int*>(sqv + 16);
  for (int idx = threadIdx.x; idx < 16 * D; idx += 256) {
    const int row = idx / D;
    qf[idx] = row < G ? a.q[((size_t)b * a.Hq + hk * G + row) * D + idx % D] : 0.0f;
  }
  __syncthreads();
  prepare_query_lds<L, D>(qf, q8, sqv, qsum);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;       // QK: head column; PV: d-row group; V octet
  const int r = lane >> 4;         // lane group: k-slot block / C rows 4r..4r+3

  // int8 query as the B operand of Q K^T, k-slot order [0,2,4,6,1,3,5,7] per 8
  uint32_t qb[NG][2];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(q8 + col * D + 32 * g + 8 * r);
    const uint32_t w0 = p[0], w1 = p[1];
    qb[g][0] = __builtin_amdgcn_perm(w1, w0, 0x06040200u);
    qb[g][1] = __builtin_amdgcn_perm(w1, w0, 0x07050301u);
  }
  int qoff[SG];      // bias * sum(q8) removed from the biased-code dot
  float qzf[SG];     // sum(q8) per block for the zero-point term
#pragma unroll
  for (int g = 0; g < SG; ++g) {
    int s = 0;
    if (L == HAD) {
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) s += qsum[col * NG + gg];
    } else {
      s = qsum[col * NG + g];
    }
    qoff[g] = BIAS * s;
    qzf[g] = (float)s;
  }
  const float sqc = sqv[col] * a.alpha * KVQ_LOG2E;
  __syncthreads();   // the LDS is reused by the merge below

  float m_run = -INFINITY, l_run = 0.0f;
  v4f oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  const size_t row_first = plane_row(a, b, hk, t_begin);

  for (int T0 = t_begin + 32 * wave; T0 < t_end; T0 += 128) {
    // ---------------- Q K^T on the int8 MFMA
    v4i acc[2][SG];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int ta = T0 + 16 * tau + col;
      const size_t rk = ta < t_end ? plane_row(a, b, hk, ta) : row_first;
      const uint8_t* kpr = a.kp + rk * T::PB;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        uint32_t lo, hi;
        if (L == Q60) {
          const uint32_t x = *reinterpret_cast<const uint32_t*>(kpr + 24 * g + 4 * r);
          const uint32_t t2 = *reinterpret_cast<const uint16_t*>(kpr + 24 * g + 16 + 2 * r);
          q6_octet(x, t2, lo, hi);
        } else {
          uint32_t x = *reinterpret_cast<const uint32_t*>(kpr + 4 * (4 * g + r));
          if (BIAS) x ^= 0x88888888u;
          lo = x & 0x0F0F0F0Fu;
          hi = (x >> 4) & 0x0F0F0F0Fu;
        }
        const long A = (long)((uint64_t)lo | ((uint64_t)hi << 32));
        const long B = (long)((uint64_t)qb[g][0] | ((uint64_t)qb[g][1] << 32));
        if (L == HAD) {
          acc[tau][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, g == 0 ? v4i{0, 0, 0, 0} : acc[tau][0], 0, 0, 0);
        } else {
          acc[tau][g] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, v4i{0, 0, 0, 0}, 0, 0, 0);
        }
      }
    }

    // ---------------- scores of this lane's 8 tokens (C rows 4r+j of both tiles)
    float xs[8];
    float vscale_had[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tb = T0 + 16 * tau + 4 * r;
      const size_t rb = tb < t_end ? plane_row(a, b, hk, tb) : row_first;
      const uint8_t* rec = a.ks + rb * T::SB;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = tb + j;
        float x = 0.0f;
        if (L == HAD) {
          const int I = acc[tau][0][j] - qoff[0];
          x = reinterpret_cast<const float*>(rec)[j] * (float)I;
          if (DBG && t < t_end && col < G)
            a.dbg[(((size_t)b * a.Hq + hk * G + col) * a.max_seq_len + t)] = I;
        } else {
#pragma unroll
          for (int g = 0; g < SG; ++g) {
            const int I = acc[tau][g][j] - qoff[g];
            if (L == ASYM) {
              const uint32_t sz = reinterpret_cast<const uint32_t*>(rec + j * T::SB)[g];
              const float s = (float)as_h2(sz)[0];
              const float z = (float)as_h2(sz)[1];
              x += s * (float)I + z * qzf[g];
            } else {
              const float s = (float)reinterpret_cast<const _Float16*>(rec + j * T::SB)[g];
              x += s * (float)I;
            }
            if (DBG && t < t_end && col < G)
              a.dbg[(((size_t)b * a.Hq + hk * G + col) * a.max_seq_len + t) * SG + g] = I;
          }
        }
        xs[tau * 4 + j] = t < t_end ? x * sqc : -INFINITY;
      }
      if (L == HAD) {
        // per-token V scale of the same 8 tokens (folded into the P operand)
        const uint8_t* vrec = a.vs + rb * T::SB;
#pragma unroll
        for (int j = 0; j < 4; ++j) vscale_had[tau * 4 + j] = reinterpret_cast<const float*>(vrec)[j];
      }
    }
    if (DBG) continue;

    // ---------------- online softmax (base 2), per head = lane column
    float smax = xs[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) smax = fmaxf(smax, xs[i]);
    smax = fmaxf(smax, __shfl_xor(smax, 16));
    smax = fmaxf(smax, __shfl_xor(smax, 32));
    const float m_new = fmaxf(m_run, smax);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float corr = exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
    v8h pB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = exp2f(xs[i] - m_use);
      psum += p;
      pB[i] = (_Float16)(L == HAD ? p * vscale_had[i] : p);
    }
    l_run = l_run * corr + psum;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[i] *= corr;

    // ---------------- P V on the f16 MFMA, V^T built from the packed rows
#pragma unroll
    for (int o = 0; o < NO; ++o) {
      const int oc = col + 16 * o;       // this lane's octet (elements 8*oc .. 8*oc+7)
      const int grp = oc >> 2;           // its 32-element block
      uint32_t ev[8], od[8];             // per token (k-slot): even / odd element codes as bytes or raw dword
      uint32_t sz[8];                    // per token: fp16 scale (| zero << 16 for ASYM)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int tb = T0 + 16 * tau + 4 * r;
        const size_t rb = tb < t_end ? plane_row(a, b, hk, tb) : row_first;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const size_t rv = (tb + j < t_end) ? rb + j : row_first;
          const uint8_t* vpr = a.vp + rv * T::PB;
          const int k = tau * 4 + j;
          if (L == Q60) {
            const uint32_t x = *reinterpret_cast<const uint32_t*>(vpr + 24 * grp + 4 * (oc & 3));
            const uint32_t t2 = *reinterpret_cast<const uint16_t*>(vpr + 24 * grp + 16 + 2 * (oc & 3));
            q6_octet(x, t2, ev[k], od[k]);
          } else {
            uint32_t x = *reinterpret_cast<const uint32_t*>(vpr + 4 * oc);
            if (BIAS) x ^= 0x88888888u;
            ev[k] = x;
            od[k] = 0;
          }
          if (L == ASYM) {
            sz[k] = reinterpret_cast<const uint32_t*>(a.vs + rv * T::SB)[grp];
          } else if (L != HAD) {
            sz[k] = reinterpret_cast<const uint16_t*>(a.vs + rv * T::SB)[grp];
          } else {
            sz[k] = 0;
          }
        }
      }
      // f16x2 scale / zero of token pairs (k-slots 2i, 2i+1)
      h2 s2[4], z2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s2[i] = as_h2(__builtin_amdgcn_perm(sz[2 * i + 1], sz[2 * i], 0x05040100u));
        z2[i] = as_h2(__builtin_amdgcn_perm(sz[2 * i + 1], sz[2 * i], 0x07060302u));
      }
      // element e of the octet -> d = 8*oc + e -> PV tile (o, e)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v8h A;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t pair;
          if (L == Q60) {
            // byte e/2 of the even/odd code dwords of tokens 2i, 2i+1
            const uint32_t src_a = (e & 1) ? od[2 * i] : ev[2 * i];
            const uint32_t src_b = (e & 1) ? od[2 * i + 1] : ev[2 * i + 1];
            const uint32_t bsel = (uint32_t)(e >> 1);
            pair = __builtin_amdgcn_perm(src_b, src_a, bsel | (0x0Cu << 8) | ((4u + bsel) << 16) | (0x0Cu << 24)) | 0x64006400u;
          } else {
            const uint32_t bsel = (uint32_t)(e >> 1);
            const uint32_t y = __builtin_amdgcn_perm(ev[2 * i + 1], ev[2 * i], bsel | (0x0Cu << 8) | ((4u + bsel) << 16) | (0x0Cu << 24));
            pair = ((e & 1) ? (y >> 4) : y) & 0x000F000Fu;
            pair |= 0x64006400u;
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
  if (DBG) return;

  // ---------------- merge the four waves of the block (fixed order)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  float* mbuf = reinterpret_cast<float*>(smem);          // [4][16]
  float* lbuf = mbuf + 64;                               // [4][16]
  float* obuf = lbuf + 64;                               // [4][G][D]
  if (r == 0) {
    mbuf[wave * 16 + col] = m_run;
    lbuf[wave * 16 + col] = l_run;
  }
  if (col < G) {
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 8 * (4 * r + j + 16 * o) + e;
          obuf[(wave * G + col) * D + d] = oacc[o * 8 + e][j];
        }
  }
  __syncthreads();
  const int PST = partial_stride(D);
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mbuf[w * 16 + h]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = mbuf[w * 16 + h];
      const float e = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
      o += e * obuf[(w * G + h) * D + d];
      l += e * lbuf[w * 16 + h];
    }
    float* dst = a.ws + (((size_t)b * a.Hq + hk * G + h) * a.nc1 + c) * PST;
    dst[d] = o;
    if (d == 0) {
      dst[D] = M;
      dst[D + 1] = l;
    }
  }
}

// Online-softmax merge of the chunk partials; Hadamard layout: rotate back.
template <int D, bool ROT>
__global__ __launch_bounds__(256) void decode_reduce(const float* ws, float* out, const int32_t* seq_len,
                                                     int Hq, int nc1, int chunk, int n_recent) {
  __shared__ float x[D];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int S = seq_len[b];
  const int Sq = n_recent > 0 ? max(0, S - n_recent) : S;
  const int nq = (Sq + chunk - 1) / chunk;
  const bool has_w = n_recent > 0 && S > 0;
  const int PST = partial_stride(D);
  const float* base = ws + ((size_t)b * Hq + h) * nc1 * PST;
  float M = -INFINITY;
  for (int c = 0; c < nq; ++c) M = fmaxf(M, base[(size_t)c * PST + D]);
  if (has_w) M = fmaxf(M, base[(size_t)(nc1 - 1) * PST + D]);
  float o = 0.0f, l = 0.0f;
  for (int c = 0; c < nq + (has_w ? 1 : 0); ++c) {
    const int cc = c < nq ? c : nc1 - 1;
    const float* p = base + (size_t)cc * PST;
    const float mc = p[D];
    const float w = (mc == -INFINITY) ? 0.0f : exp2f(mc - M);
    o += w * p[d];
    l += w * p[D + 1];
  }
  float res = l > 0.0f ? o / l : 0.0f;
  if (ROT) {
    // rotate back with the same butterfly transform (stages h = 1 .. D/2, then 1/sqrt(D))
    x[d] = res;
    __syncthreads();
    for (int hh = 1; hh < D; hh <<= 1) {
      int i = 0;
      float p = 0.0f, q = 0.0f;
      if (d < D / 2) {
        i = (d / hh) * 2 * hh + (d % hh);
        p = x[i];
        q = x[i + hh];
      }
      __syncthreads();
      if (d < D / 2) {
        x[i] = p + q;
        x[i + hh] = p - q;
      }
      __syncthreads();
    }
    res = x[d] * hadamard_norm<D>();
  }
  out[((size_t)b * Hq + h) * D + d] = res;
}

template <int L, int D, bool DBG>
static void launch_partial(const DecodeArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  if (lds > 65536)
    (void)hipFuncSetAttribute((const void*)decode_partial<L, D, DBG>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((decode_partial<L, D, DBG>), grid, dim3(256), lds, st, a);
}

typedef void (*partial_fn)(const DecodeArgs&, dim3, size_t, hipStream_t);

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

static size_t partial_lds_bytes(int D, int G, int n_recent) {
  const size_t pro = (size_t)16 * D * 4 + 16 * D + 16 * 4 + 16 * (D / 32) * 4;
  const size_t merge = 2 * 64 * 4 + (size_t)4 * G * D * 4;
  const size_t win = n_recent > 0 ? pro + (size_t)16 * n_recent * 4 + 32 * 4 : 0;
  size_t m = pro > merge ? pro : merge;
  return m > win ? m : win;
}

static int chunks_of(int max_seq_len, int chunk) { return (max_seq_len + chunk - 1) / chunk; }

static kvq_status check_attend_args(const kvq_cache* c, const void* q, int32_t batch, int32_t Hq,
                                    const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                                    int32_t max_seq_len) {
  kvq_status st = validate_cache(c);
  if (st != KVQ_OK) return st;
  if (!q || !block_table || !seq_len) return fail(KVQ_ERR_INVALID_ARG, "q, block_table and seq_len must be non-null");
  if (batch < 1) return fail(KVQ_ERR_INVALID_ARG, "batch must be >= 1");
  if (Hq < 1 || Hq % c->num_kv_heads) return fail(KVQ_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (Hq / c->num_kv_heads > 16) return fail(KVQ_ERR_UNSUPPORTED, "GQA group larger than 16 heads");
  if (max_seq_len < 0) return fail(KVQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (max_pages < 1 || (int64_t)max_pages * c->page_size < max_seq_len)
    return fail(KVQ_ERR_INVALID_ARG, "max_pages_per_seq * page_size must cover max_seq_len");
  if (c->n_recent > 512) return fail(KVQ_ERR_UNSUPPORTED, "n_recent above 512");
  return KVQ_OK;
}

}  // namespace kvq

using namespace kvq;

extern "C" size_t kvq_decode_workspace_bytes(int32_t batch, int32_t Hq, int32_t D, int32_t max_seq_len,
                                             int32_t chunk) {
  if (batch < 1 || Hq < 1 || (D != 128 && D != 256) || max_seq_len < 0 || chunk < 128 || chunk % 128) return 0;
  // +1 slot for the window partial (always reserved so the size does not depend on n_recent)
  const size_t nc1 = (size_t)chunks_of(max_seq_len, chunk) + 1;
  return (size_t)batch * Hq * nc1 * partial_stride(D) * sizeof(float);
}

extern "C" kvq_status kvq_attend_decode(const kvq_cache* c, const float* q, float* out, int32_t batch, int32_t Hq,
                                        float alpha, const int32_t* block_table, int32_t max_pages,
                                        const int32_t* seq_len, int32_t max_seq_len, int32_t chunk,
                                        void* workspace, size_t ws_bytes, void* stream) {
  kvq_status st = check_attend_args(c, q, batch, Hq, block_table, max_pages, seq_len, max_seq_len);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out must be non-null");
  if (chunk < 128 || chunk % 128) return fail(KVQ_ERR_INVALID_ARG, "chunk_tokens must be a positive multiple of 128");
  const size_t need = kvq_decode_workspace_bytes(batch, Hq, c->head_dim, max_seq_len, chunk);
  if (!workspace || ws_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  const int D = c->head_dim;
  DecodeArgs a;
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
  a.dbg = nullptr;
  a.Hkv = c->num_kv_heads;
  a.Hq = Hq;
  a.G = Hq / c->num_kv_heads;
  a.page_shift = __builtin_ctz((unsigned)c->page_size);
  a.n_recent = c->n_recent;
  a.max_pages = max_pages;
  a.chunk = chunk;
  const int nch = chunks_of(max_seq_len, chunk);
  a.nc1 = nch + 1;
  a.max_seq_len = max_seq_len;
  a.alpha = alpha;
  hipStream_t s = (hipStream_t)stream;
  const int gx = nch + (c->n_recent > 0 ? 1 : 0);
  if (gx > 0) {
    const dim3 grid(gx, c->num_kv_heads, batch);
    pick_partial<false>(c->layout, D)(a, grid, partial_lds_bytes(D, a.G, c->n_recent), s);
    st = check_launch("decode partial kernel");
    if (st != KVQ_OK) return st;
  }
  const dim3 rgrid(Hq, batch);
  const bool rot = c->layout == HAD;
  if (D == 128) {
    if (rot) hipLaunchKernelGGL((decode_reduce<128, true>), rgrid, dim3(128), 0, s, a.ws, out, seq_len, Hq, a.nc1, chunk, c->n_recent);
    else hipLaunchKernelGGL((decode_reduce<128, false>), rgrid, dim3(128), 0, s, a.ws, out, seq_len, Hq, a.nc1, chunk, c->n_recent);
  } else {
    if (rot) hipLaunchKernelGGL((decode_reduce<256, true>), rgrid, dim3(256), 0, s, a.ws, out, seq_len, Hq, a.nc1, chunk, c->n_recent);
    else hipLaunchKernelGGL((decode_reduce<256, false>), rgrid, dim3(256), 0, s, a.ws, out, seq_len, Hq, a.nc1, chunk, c->n_recent);
  }
  return check_launch("decode reduce kernel");
}

extern "C" kvq_status kvq_debug_qk_i32(const kvq_cache* c, const float* q, int32_t batch, int32_t Hq,
                                       const int32_t* block_table, int32_t max_pages, const int32_t* seq_len,
                                       int32_t max_seq_len, int32_t* scores, void* stream) {
  kvq_status st = check_attend_args(c, q, batch, Hq, block_table, max_pages, seq_len, max_seq_len);
  if (st != KVQ_OK) return st;
  if (!scores) return fail(KVQ_ERR_INVALID_ARG, "scores must be non-null");
  const int chunk = 512;
  const int nch = chunks_of(max_seq_len, chunk);
  if (nch == 0) return KVQ_OK;
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.kp = (const uint8_t*)c->k_payload;
  a.vp = (const uint8_t*)c->v_payload;
  a.ks = (const uint8_t*)c->k_scale;
  a.vs = (const uint8_t*)c->v_scale;
  a.q = q;
  a.block_table = block_table;
  a.seq_len = seq_len;
  a.dbg = scores;
  a.Hkv = c->num_kv_heads;
  a.Hq = Hq;
  a.G = Hq / c->num_kv_heads;
  a.page_shift = __builtin_ctz((unsigned)c->page_size);
  a.n_recent = c->n_recent;
  a.max_pages = max_pages;
  a.chunk = chunk;
  a.nc1 = nch;
  a.max_seq_len = max_seq_len;
  a.alpha = 1.0f;
  const dim3 grid(nch, c->num_kv_heads, batch);
  pick_partial<true>(c->layout, c->head_dim)(a, grid, partial_lds_bytes(c->head_dim, a.G, 0), (hipStream_t)stream);
  return check_launch("score export kernel");
}
