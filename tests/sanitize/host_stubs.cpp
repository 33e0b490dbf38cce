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

}  // namespace pda

// The allocation-free call without its per-device scratch array: a call that
// needs workspace reports the missing device code; one that needs none (no
// work, or an unsplit plan) goes on as in the library.
extern "C" int32_t pda_paged_decode_attn_noalloc(const void* q, const void* k_cache,
                                                 const void* v_cache, const int32_t* block_table,
                                                 const int32_t* context_lens, float scale,
                                                 void* out, const pda_attn_desc* d,
                                                 void* stream) {
    size_t need = 0;
    const int32_t rc = pda_attn_workspace_size(d, &need);
    if (rc != PDA_OK) return rc;
    if (need > 0) {
        pda::set_error("host-only build: no device code");
        return PDA_EHIP;
    }
    return pda_paged_decode_attn(q, k_cache, v_cache, block_table, context_lens, scale, out, d,
                                 nullptr, 0, stream);
}
