// host_only_launchers.cpp -- every launcher of kvq_internal.h, launching nothing: linked
// only into the host-validation build (build.build_host_checked), where the C ABI's
// argument checks run under AddressSanitizer and UndefinedBehaviorSanitizer with no GPU
// code at all. A call that passes validation there does nothing and returns KVQ_OK.
#include "kvq_internal.h"

namespace kvq {

namespace {
hipError_t none() { return hipSuccess; }
}  // namespace

hipError_t launch_quantize_pack(int, int, const uint16_t *, int64_t, int32_t, int64_t, int64_t,
                                uint8_t *, int64_t, int32_t, int32_t, int32_t, int32_t,
                                hipStream_t) { return none(); }
hipError_t launch_decode(const DecodeParams &, hipStream_t) { return none(); }
hipError_t launch_decode_fused(const DecodeParams &, hipStream_t) { return none(); }
hipError_t launch_decode_fused_noalloc(DecodeParams, hipStream_t) { return none(); }
hipError_t launch_decode_paged_fused(const DecodeParams &, hipStream_t) { return none(); }
hipError_t launch_decode_valu(const DecodeParams &, hipStream_t) { return none(); }
hipError_t launch_decode_paged(const DecodeParams &, hipStream_t) { return none(); }
hipError_t launch_decode_outer(const DecodeParams &, hipStream_t) { return none(); }
hipError_t launch_quantize_pack_outer(int, const uint16_t *, int64_t, int32_t, int64_t, int64_t,
                                      uint8_t *, int64_t, int32_t, int32_t, int32_t,
                                      hipStream_t) { return none(); }
hipError_t launch_decode_f16(const DecodeParams &, hipStream_t) { return none(); }
hipError_t launch_combine(const float *, const float *, int32_t, int32_t, int32_t, void *, int32_t,
                          hipStream_t) { return none(); }
hipError_t launch_stream_read(const void *const *, const int64_t *, int32_t, uint32_t *,
                              hipStream_t) { return none(); }
hipError_t launch_append(const uint16_t *, const uint16_t *, uint16_t *, uint16_t *, int32_t,
                         int32_t, int32_t, int32_t, hipStream_t) { return none(); }
hipError_t launch_pack_tokens_paged(const PagedPool &, const uint16_t *, int32_t, int32_t, int64_t,
                                    int64_t, const int32_t *, const int32_t *, int32_t, uint8_t *,
                                    hipStream_t) { return none(); }
hipError_t launch_copy_state(int32_t *, const int32_t *, int32_t, hipStream_t) { return none(); }
hipError_t launch_append_evict(const PagedPool &, const uint16_t *, const uint16_t *, uint16_t *,
                               uint16_t *, int32_t, int32_t, uint8_t *, uint8_t *, int32_t *,
                               int32_t, int32_t, hipStream_t) { return none(); }
hipError_t launch_key_norm(const uint16_t *, int64_t, int32_t, int64_t, int64_t, float *,
                           hipStream_t) { return none(); }
hipError_t launch_channel_scale(const uint16_t *, int64_t, int32_t, int64_t, int64_t, const float *,
                                int64_t, int, uint16_t *, int64_t, int64_t,
                                hipStream_t) { return none(); }

}  // namespace kvq
