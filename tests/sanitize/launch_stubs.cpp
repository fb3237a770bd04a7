// launch_stubs.cpp -- stand-ins for the device-side launchers of libpkvs, so
// that its host code (plan.cpp, run.cpp) can be built for the CPU alone with
// the address and undefined-behaviour sanitizers and driven by the host tests.
// Test infrastructure: never part of the product library.  Without a GPU the
// host code only makes dry plans and rejects run calls before any launch; a
// launch that is reached anyway reports hipErrorNoDevice.
#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

#include "../../paged_kv_sliding_amd/csrc/pkvs_internal.h"

namespace pkvs {

hipError_t launch_prefill_16bit(const PrefillArgs &, int, int, bool, int, int, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_attention_fp32(const PrefillArgs &, int, int, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_decode_16bit(const DecodeArgs &, int, bool, int, int, int, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_decode_merge(const DecodeArgs &, int, bool, bool, int, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_merge_state(const void *, const float *, const void *, const float *, void *,
                              float *, int64_t, int32_t, int32_t, int32_t, int, hipStream_t)
{
    return hipErrorNoDevice;
}
int merge_state_vec_chunks(int32_t, int32_t) { return 0; }
hipError_t launch_merge_state_vec(const void *, const float *, const void *, const float *,
                                  void *, float *, int64_t, int32_t, int32_t, int32_t, int,
                                  hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_append_kv(const void *, const void *, const int64_t *, int64_t, int64_t, void *,
                            void *, int64_t, int32_t *, int, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_append_kv_quant(const void *, const void *, const int64_t *, int64_t, int64_t,
                                  int, int, void *, void *, int64_t, float, float, int32_t *, int,
                                  hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_build_kv_indices(const int32_t *, int64_t, int64_t, const int32_t *,
                                   const int32_t *, const int32_t *, int32_t, int32_t *, int32_t *,
                                   int64_t, int32_t *, int, hipStream_t)
{
    return hipErrorNoDevice;
}
int prefill_blocks_per_cu(int, int, bool, int, int) { return 0; }
int decode_blocks_per_cu(int, bool, int, int) { return 0; }

hipError_t scratch_for_device(int, void **ptr)
{
    *ptr = nullptr;
    return hipErrorNoDevice;
}

}  // namespace pkvs
