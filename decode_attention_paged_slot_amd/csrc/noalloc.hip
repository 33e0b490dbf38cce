// noalloc.hip -- paged decode attention for callers that cannot allocate:
// the split-KV workspace comes from a fixed device array of this library
// instead of the caller.
//
// `scratch` is a file-scope device array. In host code its name is only a
// stand-in for the symbol, not a device address: every device holds its own
// copy at its own address, which hipGetSymbolAddress reports once per device
// (with that device current) and which is kept here. Host code uses only
// that pointer.
#include <mutex>

#include <hip/hip_runtime.h>

#include "pda.h"
#include "pda_internal.h"

namespace pda {

namespace {

constexpr size_t kScratchBytes = PDA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (resolved on the first call on that
// device), or nullptr with the error recorded.
void* scratch_for_current_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        set_error("noalloc: no usable current device (%s)",
                  e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            set_error("noalloc: hipGetSymbolAddress: %s",
                      e != hipSuccess ? hipGetErrorString(e) : "null address");
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

}  // namespace pda

extern "C" {

int32_t pda_paged_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* context_lens,
                                      float scale, void* out, const pda_attn_desc* d,
                                      void* stream) {
    size_t need = 0;
    int32_t rc = pda_attn_workspace_size(d, &need);
    if (rc != PDA_OK) return rc;
    if (need > pda::kScratchBytes) {
        pda::set_error("noalloc: this call needs %zu bytes of workspace, above the %zu-byte "
                       "limit of the library's fixed scratch (use pda_paged_decode_attn with a "
                       "caller workspace)",
                       need, pda::kScratchBytes);
        return PDA_EWORKSPACE;
    }
    void* ws = nullptr;
    if (need > 0) {
        ws = pda::scratch_for_current_device();
        if (ws == nullptr) return PDA_EHIP;
    }
    return pda_paged_decode_attn(q, k_cache, v_cache, block_table, context_lens, scale, out, d,
                                 ws, need, stream);
}

}  // extern "C"
