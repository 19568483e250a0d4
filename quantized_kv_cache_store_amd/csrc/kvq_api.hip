// Host side of the C ABI: validation, error strings, sizing.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>

#include "kvq_internal.h"

namespace kvq {

static thread_local char g_err[512] = "";

kvq_status fail(kvq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

kvq_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return KVQ_OK;
}

int device_cus() {
  static std::atomic<int> cus_of[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cus = cus_of[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    cus_of[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

kvq_status validate_cache(const kvq_cache* c) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache descriptor is null");
  if (c->layout < 0 || c->layout >= kNumLayouts) return fail(KVQ_ERR_INVALID_ARG, "unknown layout %d", c->layout);
  if (c->head_dim != 128 && c->head_dim != 256)
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d (supported: 128, 256)", c->head_dim);
  if (c->num_kv_heads < 1) return fail(KVQ_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (c->page_size < 16 || (c->page_size & (c->page_size - 1)))
    return fail(KVQ_ERR_INVALID_ARG, "page_size must be a power of two >= 16");
  if (c->num_pages < 1) return fail(KVQ_ERR_INVALID_ARG, "num_pages must be >= 1");
  if ((int64_t)c->num_pages * c->page_size > (int64_t)INT32_MAX)
    return fail(KVQ_ERR_INVALID_ARG, "num_pages * page_size must fit the int32 slot index");
  if (c->n_recent < 0) return fail(KVQ_ERR_INVALID_ARG, "n_recent must be >= 0");
  if (c->reserved != 0) return fail(KVQ_ERR_INVALID_ARG, "reserved field must be 0");
  if (!c->k_payload || !c->v_payload || !c->k_scale || !c->v_scale)
    return fail(KVQ_ERR_INVALID_ARG, "payload and scale planes must be non-null");
  if (c->n_recent > 0 && (c->max_batch < 1 || !c->k_recent || !c->v_recent))
    return fail(KVQ_ERR_INVALID_ARG, "n_recent > 0 needs max_batch >= 1 and both window rings");
  return KVQ_OK;
}

}  // namespace kvq

using namespace kvq;

extern "C" size_t kvq_payload_bytes(int32_t layout, int32_t head_dim) { return payload_bytes_rt(layout, head_dim); }

extern "C" size_t kvq_scale_bytes(int32_t layout, int32_t head_dim) { return scale_bytes_rt(layout, head_dim); }

extern "C" const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

extern "C" const char* kvq_last_error(void) { return g_err; }
