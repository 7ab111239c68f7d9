// Randomized factorisation of the heads-merged K and V (placeholder until the
// device compressor lands: loading factors through ap_cache_set_factors works).
#include "ap_internal.h"

namespace ap {

hipError_t run_compress(ap_cache* c, const void* k, const void* v, hipStream_t st) {
  (void)c; (void)k; (void)v; (void)st;
  set_error("the device compressor is not built yet; load factors with ap_cache_set_factors");
  return hipErrorNotSupported;
}

}  // namespace ap
