// host_stubs.cpp -- device-side entry points replaced by stubs, so the
// library's host code (block pool, descriptor checks, split plan, workspace
// layout, argument validation of every call) builds with the host compiler
// alone and runs under AddressSanitizer / UndefinedBehaviorSanitizer on a
// machine without a GPU. Each stub reports that no device code is present;
// the tests that use this build make no device call.
#include <hip/hip_runtime.h>

#include "pda.h"
#include "pda_internal.h"

namespace pda {

hipError_t launch_attn_mfma(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_f32(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_prefix(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_append(const AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_append_quant(const AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_append_int4(const void*, const void*, const int32_t*, const int32_t*, void*,
                              void*, const float*, float*, void*, void*, int32_t, int32_t,
                              int32_t, int32_t, int32_t, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_merge_for_attn(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_merge_stream(const AttnArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_lse_merge(const float*, const float*, int32_t, int32_t, int32_t, float*,
                            hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_read_probe(const void*, size_t, const int64_t*, int64_t, int32_t, int32_t,
                             uint32_t*, hipStream_t) {
    return hipErrorNoDevice;
}
size_t attn_mfma_dyn_lds(int32_t B) { return (size_t)(3 * B + 2) * sizeof(int32_t); }

}  // namespace pda

extern "C" int32_t pda_paged_decode_attn_noalloc(const void*, const void*, const void*,
                                                 const int32_t*, const int32_t*, float, void*,
                                                 const pda_attn_desc*, void*) {
    pda::set_error("host-only build: no device code");
    return PDA_EHIP;
}
