// Chunked-prefill attention (MFMA).  Placeholder entry point until the kernel
// lands: validates nothing and reports the configuration as not built.
#include "pkv_device.h"
#include "pkv_internal.h"

extern "C" int paged_attention_prefill_chunk(void*, int32_t, const void*, const void*, const void*,
                                             const int32_t*, int32_t, const int32_t*, const int32_t*,
                                             int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                                             int32_t, int64_t, int32_t, float, int32_t, void*) {
  return pkv::fail(PKV_EUNSUPPORTED, "paged_attention_prefill_chunk: not built yet");
}
