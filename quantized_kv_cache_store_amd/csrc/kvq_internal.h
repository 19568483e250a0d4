// Internal definitions shared by the libkvq translation units (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/kvq.h"

namespace kvq {

enum : int { HAD = KVQ_LAYOUT_HAD_INT4, Q40 = KVQ_LAYOUT_Q4_0, Q60 = KVQ_LAYOUT_Q6_0, ASYM = KVQ_LAYOUT_ASYM_INT4_G32 };

// Per-(layout, head_dim) constants of one stored row.
template <int L, int D>
struct Layout {
  static_assert(D == 128 || D == 256, "head_dim 128 or 256");
  static constexpr int NG = D / 32;                                   // 32-element blocks
  static constexpr int PB = (L == Q60) ? NG * 24 : D / 2;             // payload bytes
  static constexpr int SB = (L == HAD) ? 4 : (L == ASYM ? NG * 4 : NG * 2);  // record bytes
  static constexpr int SG = (L == HAD) ? 1 : NG;                      // scale groups
  static constexpr int OCT = D / 8;                                   // 8-element octets
};

// Offset added to a signed code to make it non-negative (n + OFF = code ^ OFF).
template <int L>
struct CodeBias {
  static constexpr int value = (L == Q60) ? 32 : (L == ASYM ? 0 : 8);
};

static inline size_t payload_bytes_rt(int layout, int D) {
  if ((D != 128 && D != 256) || layout < 0 || layout > 3) return 0;
  return layout == Q60 ? (size_t)(D / 32) * 24 : (size_t)D / 2;
}
static inline size_t scale_bytes_rt(int layout, int D) {
  if ((D != 128 && D != 256) || layout < 0 || layout > 3) return 0;
  if (layout == HAD) return 4;
  return layout == ASYM ? (size_t)(D / 32) * 4 : (size_t)(D / 32) * 2;
}

// Split-K partial record: o[D] (unnormalised), m (base-2 logit max), l, 2 pad.
static inline constexpr int partial_stride(int D) { return D + 4; }

// host-side error reporting (kvq_api.hip)
kvq_status fail(kvq_status s, const char* fmt, ...);
kvq_status check_launch(const char* what);
kvq_status validate_cache(const kvq_cache* c);

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
// ----------------------------------------------------------------------------- device helpers

// 1/sqrt(D) rounded to f32: D=128 -> 0x3db504f3, D=256 -> 1/16.
template <int D>
__device__ __forceinline__ float hadamard_norm() {
  return D == 128 ? 0x1.6a09e6p-4f : 0.0625f;
}

__device__ __forceinline__ float wave_max16(float v) {
  // max over the 16-lane row that holds this lane (lanes 16r..16r+15)
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}

// Query preparation in LDS for up to 16 vectors of length D, by a 256-thread block.
//   qf    f32 [16][D]: input, replaced by the f32 query the window uses (rotated for HAD)
//   q8    int8 [16][D]: out, per-vector symmetric int8 with sq = amax / 127
//   sq    f32 [16]
//   qsum  int32 [16][D/32]: sum of q8 over each 32-element block
// Rows past n_rows must hold zeros on entry (they give q8 = 0, sq = 0).
// The rotation is the butterfly transform with stages h = 1, 2, 4, ..., D/2,
// each butterfly (a, b) -> (a + b, a - b) in f32, then every element times
// f32(1/sqrt(D)); every value is an IEEE f32 result, so the order in which
// threads run the independent butterflies does not change it.
template <int L, int D>
__device__ void prepare_query_lds(float* qf, int8_t* q8, float* sq, int* qsum) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x;
  constexpr int R = 16;
  if (L == HAD) {
    for (int h = 1; h < D; h <<= 1) {
      for (int idx = tid; idx < R * D / 2; idx += 256) {
        const int row = idx / (D / 2), k = idx % (D / 2);
        const int i = (k / h) * 2 * h + (k % h);
        float* x = qf + row * D;
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
      __syncthreads();
    }
    for (int idx = tid; idx < R * D; idx += 256) qf[idx] = qf[idx] * hadamard_norm<D>();
    __syncthreads();
  }
  // amax per row: 16 threads per row
  {
    const int row = tid >> 4, sub = tid & 15;
    float m = 0.0f;
    for (int d = sub; d < D; d += 16) m = fmaxf(m, fabsf(qf[row * D + d]));
    m = wave_max16(m);
    if (sub == 0) sq[row] = m / 127.0f;
  }
  __syncthreads();
  for (int idx = tid; idx < R * D; idx += 256) {
    const float s = sq[idx / D];
    int v = 0;
    if (s != 0.0f) v = (int)fminf(fmaxf(rintf(qf[idx] / s), -127.0f), 127.0f);
    q8[idx] = (int8_t)v;
  }
  __syncthreads();
  for (int idx = tid; idx < R * (D / 32); idx += 256) {
    const int row = idx / (D / 32), g = idx % (D / 32);
    int acc = 0;
    for (int j = 0; j < 32; ++j) acc += q8[row * D + g * 32 + j];
    qsum[idx] = acc;
  }
  __syncthreads();
}
#endif

}  // namespace kvq
