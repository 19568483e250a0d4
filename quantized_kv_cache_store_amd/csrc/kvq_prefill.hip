// Causal prefill over the packed cache (placeholder until the tiled kernel lands).
#include "kvq_internal.h"

using namespace kvq;

extern "C" size_t kvq_prefill_workspace_bytes(int32_t, int32_t, int32_t, int32_t, int32_t) { return 0; }

extern "C" kvq_status kvq_attend_prefill_causal(const kvq_cache*, const float*, float*, int32_t, int32_t, int32_t,
                                                float, int32_t, const int32_t*, const int32_t*, int32_t,
                                                const int32_t*, int32_t, uint32_t, void*, size_t, void*) {
  return fail(KVQ_ERR_UNSUPPORTED, "causal prefill is not built yet");
}
