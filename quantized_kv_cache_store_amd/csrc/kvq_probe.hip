// Read-only streaming probe: the rate at which the device reads buffers from HBM through the same
// direct-to-LDS 16-byte nontemporal loads the decode kernel streams its cache with, many in flight
// per wave.  It gives the attainable read rate that the decode kernel's HBM rate is compared with
// (next to the nominal 8 TB/s).  The loaded data lands in a per-wave LDS slot that nothing reads.

#include "kvq_internal.h"

namespace kvq {

constexpr int kProbeBufs = 4;

struct ProbeArgs {
  const uint8_t* src[kProbeBufs];
  size_t bytes[kProbeBufs];
  size_t first[kProbeBufs + 1];   // first 1 KiB piece of each buffer in the joint numbering
  size_t per;                     // pieces per wave
};

__device__ __forceinline__ void probe_dma16(const uint8_t* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" : : "v"(src), "{m0}"(lds) : "memory");
}

// The buffers' 1 KiB pieces are numbered one after the other; wave w of the grid reads pieces
// [w * per, (w + 1) * per) (a buffer's last piece may be partial: its lanes past the end stay idle),
// up to 16 in flight.
__global__ __launch_bounds__(256) void stream_read(ProbeArgs a) {
  __shared__ __align__(16) unsigned char slot[4 * 1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(slot + wave * 1024));
  const size_t w = (size_t)blockIdx.x * 4 + wave;
  const size_t total = a.first[kProbeBufs];
  const size_t p0 = w * a.per, p1 = p0 + a.per < total ? p0 + a.per : total;
  int issued = 0;
#pragma unroll
  for (int i = 0; i < kProbeBufs; ++i) {   // the part of [p0, p1) in buffer i (static indices: no scratch)
    const size_t lo = p0 > a.first[i] ? p0 : a.first[i];
    const size_t hi = p1 < a.first[i + 1] ? p1 : a.first[i + 1];
    for (size_t p = lo; p < hi; ++p) {
      const size_t off = (p - a.first[i]) * 1024 + (size_t)lane * 16;
      if (off < a.bytes[i]) probe_dma16(a.src[i] + off, lds);
      if (++issued == 8) {
        asm volatile("s_waitcnt vmcnt(8)" : : : "memory");
        issued = 0;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
}

}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_debug_stream_read(int32_t n, const void* const* src, const size_t* bytes, void* stream) {
  if (n < 1 || n > kProbeBufs || !src || !bytes) return fail(KVQ_ERR_INVALID_ARG, "1 to %d buffers", kProbeBufs);
  ProbeArgs a;
  memset(&a, 0, sizeof(a));
  size_t pieces = 0;
  for (int i = 0; i < kProbeBufs; ++i) {
    a.first[i] = pieces;
    if (i >= n) continue;
    if (!src[i]) return fail(KVQ_ERR_INVALID_ARG, "src[%d] is null", i);
    if (bytes[i] % 16 || ((uintptr_t)src[i] & 15)) return fail(KVQ_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
    a.src[i] = (const uint8_t*)src[i];
    a.bytes[i] = bytes[i];
    pieces += (bytes[i] + 1023) / 1024;
  }
  a.first[kProbeBufs] = pieces;
  if (pieces == 0) return KVQ_OK;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  const size_t blocks = (size_t)cus * 8, waves = blocks * 4;
  a.per = (pieces + waves - 1) / waves;
  hipLaunchKernelGGL(stream_read, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return check_launch("stream probe kernel");
}
