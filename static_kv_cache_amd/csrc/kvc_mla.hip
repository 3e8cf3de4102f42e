// Latent (MLA) decode kernels. Not built yet: every launcher reports
// "not supported", and kvc_alloc refuses MLA descriptors before reaching them.
#include "kvc_internal.h"

hipError_t kvc_launch_mla_attn(const kvc_cache*, const void*, const void*, void*, const int32_t*,
                               const int32_t*, float, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t kvc_launch_mla_absorb(const kvc_cache*, const void*, const void*, const void*, uint16_t*,
                                 hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t kvc_launch_mla_uproj(const kvc_cache*, const uint16_t*, const void*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
