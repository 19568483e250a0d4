// The decode without a workspace (kvq_attend_decode_noalloc): the kernels of kvq_attend_decode, with
// the split-K partials in a device array of this library instead of a caller's workspace.
//
// The array lives in this translation unit on purpose, apart from the attention kernels: with a
// 32 MiB array in their own code object, the decode partial kernel measured about 10 % slower (the
// same machine code, 286 against 258 us on the 128K batch-8 layer).

#include <atomic>

#include "kvq_attend_common.h"

using namespace kvq;

// The split-K partials of kvq_attend_decode_noalloc live in this file-scope device array, one copy
// per device, held from the library's load until the process ends.  Host code never passes the
// array's name to a kernel (on the host it stands for a host-side shadow, not device memory): the
// device address comes from hipGetSymbolAddress, once per device, with that device current.  The
// kernels overwrite every slot the reduce reads, so nothing in it needs clearing between calls.
namespace {
constexpr size_t kNoAllocScratchBytes = KVQ_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

kvq_status scratch_address(void** out) {
  static std::atomic<void*> addr_of[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(KVQ_ERR_HIP, "no current device below %d for the decode scratch", kMaxDevices);
  void* p = addr_of[dev].load(std::memory_order_acquire);
  if (!p) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVQ_ERR_HIP, "hipGetSymbolAddress of the decode scratch on device %d: %s", dev, hipGetErrorString(e));
    addr_of[dev].store(p, std::memory_order_release);   // racing first calls store the same address
  }
  *out = p;
  return KVQ_OK;
}
}  // namespace

extern "C" kvq_status kvq_attend_decode_noalloc(const kvq_cache* c, const float* q, float* out, int32_t batch,
                                                int32_t Hq, float alpha, const int32_t* block_table,
                                                int32_t max_pages, const int32_t* seq_len, int32_t max_seq_len,
                                                int32_t chunk, void* stream) {
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out must be non-null");
  kvq_status st = decode_check(c, q, batch, Hq, block_table, max_pages, seq_len, max_seq_len, chunk);
  if (st != KVQ_OK) return st;
  const size_t need = decode_partials_bytes(c, batch, Hq, max_seq_len, chunk);
  if (need > kNoAllocScratchBytes)
    return fail(KVQ_ERR_WORKSPACE, "this decode needs %zu bytes of partials, above the %zu-byte scratch of "
                "kvq_attend_decode_noalloc (use kvq_attend_decode with a workspace)", need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != KVQ_OK) return st;
  if ((st = decode_partial_ws(c, q, batch, Hq, alpha, block_table, max_pages, seq_len, max_seq_len, chunk, ws, stream,
                              false)) != KVQ_OK)
    return st;
  return decode_reduce_ws(c, out, batch, Hq, seq_len, max_seq_len, chunk, ws, stream);
}
