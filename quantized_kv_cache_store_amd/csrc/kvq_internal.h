// Internal definitions shared by the libkvq translation units (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/kvq.h"

namespace kvq {

enum : int {
  HAD = KVQ_LAYOUT_HAD_INT4,
  Q40 = KVQ_LAYOUT_Q4_0,
  Q60 = KVQ_LAYOUT_Q6_0,
  ASYM = KVQ_LAYOUT_ASYM_INT4_G32,
  Q80 = KVQ_LAYOUT_Q8_0
};
constexpr int kNumLayouts = 5;

// Per-(layout, head_dim) constants of one stored row.
template <int L, int D>
struct Layout {
  static_assert(D == 128 || D == 256, "head_dim 128 or 256");
  static constexpr int NG = D / 32;                                   // 32-element blocks
  static constexpr int PB = (L == Q60) ? NG * 24 : (L == Q80 ? D : D / 2);   // payload bytes
  static constexpr int SB = (L == HAD) ? 4 : (L == ASYM ? NG * 4 : NG * 2);  // record bytes
  static constexpr int SG = (L == HAD) ? 1 : NG;                      // scale groups
  static constexpr int OCT = D / 8;                                   // 8-element octets
};

// Offset added to a signed code to make it non-negative (n + OFF = code ^ OFF), the form in which
// the V side turns codes into fp16.  The K side's int8 MFMA takes the 8-bit codes as they are
// (signed), so that layout's K codes carry no offset (k_side).
template <int L>
struct CodeBias {
  static constexpr int value = (L == Q60) ? 32 : (L == ASYM ? 0 : (L == Q80 ? 128 : 8));
  static constexpr int k_side = (L == Q80) ? 0 : value;
};

static inline size_t payload_bytes_rt(int layout, int D) {
  if ((D != 128 && D != 256) || layout < 0 || layout >= kNumLayouts) return 0;
  if (layout == Q80) return (size_t)D;
  return layout == Q60 ? (size_t)(D / 32) * 24 : (size_t)D / 2;
}
static inline size_t scale_bytes_rt(int layout, int D) {
  if ((D != 128 && D != 256) || layout < 0 || layout >= kNumLayouts) return 0;
  if (layout == HAD) return 4;
  return layout == ASYM ? (size_t)(D / 32) * 4 : (size_t)(D / 32) * 2;
}

// Split-K partial record: o[D] (unnormalised), m (base-2 logit max), l, 2 pad.
static inline constexpr int partial_stride(int D) { return D + 4; }
// The prefill's partial record, in floats: D f16 values h[d], then m, l (f32) and an int exponent x;
// the unnormalised o[d] is h[d] * 2^x, the row scaled so that max |h| lies in [2^14, 2^15).  2 D + 16
// bytes: half the f32 record's, which the prefill's reduce reads and its partial kernels write.
static inline constexpr int narrow_stride(int D) { return D / 2 + 4; }

// host-side error reporting (kvq_api.hip)
kvq_status fail(kvq_status s, const char* fmt, ...);
kvq_status check_launch(const char* what);
kvq_status validate_cache(const kvq_cache* c);
// Compute units of the current device, cached per device (256 if the query fails).  Safe to call
// from several host threads: the cache entries are atomics, and racing first calls store the same
// value.
int device_cus();

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
// ----------------------------------------------------------------------------- device helpers

// 1/sqrt(D) rounded to f32: D=128 -> 0x3db504f3, D=256 -> 1/16.
template <int D>
__device__ __forceinline__ float hadamard_norm() {
  return D == 128 ? 0x1.6a09e6p-4f : 0.0625f;
}

// Maximum of two values that are never NaN, as one v_max_f32.  For fmaxf the compiler quiets each operand
// it cannot prove canonical (a value loaded from memory or moved across lanes) with an extra v_max_f32,
// and it folds a median with +inf back into that form; an instruction written out is left as it is.
__device__ __forceinline__ float fmax_nc(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// Maximum of two non-negative values, by their bit patterns (whose order is that of the values).
__device__ __forceinline__ float fmax_pos(float a, float b) {
  return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
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
// Rows past n_rows must hold zeros on entry (they give q8 = 0, sq = 0).  The caller
// synchronises the block after filling qf; this routine ends with a block barrier.
// Thread (row = tid / 16, j = tid % 16) holds elements j*E .. j*E + E - 1 of its row in
// registers.  The rotation is the butterfly transform with stages h = 1, 2, 4, ..., D/2, each
// butterfly (a, b) -> (a + b, a - b) in f32 (stages below E inside the thread, the others
// between the 16 lanes of the row), then every element times f32(1/sqrt(D)).
template <int L, int D>
__device__ void prepare_query_lds(float* qf, int8_t* q8, float* sq, int* qsum) {
#pragma clang fp contract(off)
  constexpr int E = D / 16;          // elements per thread
  constexpr int LPG = 32 / E;        // lanes per 32-element block
  const int tid = threadIdx.x;
  const int row = tid >> 4, j = tid & 15;
  float* xr = qf + row * D + j * E;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    const float4 v = *reinterpret_cast<const float4*>(xr + e);
    x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
  }
  if (L == HAD) {
#pragma unroll
    for (int hh = 1; hh < E; hh <<= 1) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if ((i & hh) == 0) {
          const float p = x[i], q = x[i + hh];
          x[i] = p + q;
          x[i + hh] = p - q;
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      const bool upper = (j & m) != 0;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const float y = __shfl_xor(x[i], m);
        x[i] = upper ? (y - x[i]) : (x[i] + y);
      }
    }
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = x[i] * hadamard_norm<D>();
#pragma unroll
    for (int e = 0; e < E; e += 4) *reinterpret_cast<float4*>(xr + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(x[i]));
  m = wave_max16(m);
  const float s = m / 127.0f;
  int gs = 0;
  uint32_t packed[E / 4];
#pragma unroll
  for (int i = 0; i < E / 4; ++i) packed[i] = 0u;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const int v = s != 0.0f ? (int)fminf(fmaxf(rintf(x[i] / s), -127.0f), 127.0f) : 0;
    gs += v;
    packed[i >> 2] |= (uint32_t)(v & 0xFF) << (8 * (i & 3));
  }
#pragma unroll
  for (int i = 0; i < E / 4; ++i) reinterpret_cast<uint32_t*>(q8 + row * D + j * E)[i] = packed[i];
#pragma unroll
  for (int o = 1; o < LPG; o <<= 1) gs += __shfl_xor(gs, o);
  if (j % LPG == 0) qsum[row * (D / 32) + j / LPG] = gs;
  if (j == 0) sq[row] = s;
  __syncthreads();
}
#endif

}  // namespace kvq
