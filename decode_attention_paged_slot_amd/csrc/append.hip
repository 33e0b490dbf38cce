// append.hip -- the append path: each new token's K and V rows land in their
// mapped cache slots ("9 Decode and KV Cache", section 9.4, append path; the
// slot of a logical position is table[pos / bs] * bs + pos % bs, section 9.5).
//
// One thread moves 16 bytes. Threads of a token are contiguous over
// (head, 16-byte chunk), so every 256-B cache row is written by 16 lanes with
// full-width stores; K and V are the two halves of grid.z.
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

__global__ void __launch_bounds__(256) k_append_copy(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int64_t* __restrict__ slots, int32_t T, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, int32_t n_kv, int32_t chunks_per_row, int32_t bs,
    int64_t num_slots) {
    const int32_t t = blockIdx.y;
    const int32_t c = blockIdx.x * blockDim.x + threadIdx.x;   // over n_kv * chunks_per_row
    if (t >= T || c >= n_kv * chunks_per_row) return;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) return;
    const int32_t head = c / chunks_per_row;
    const int32_t cr = c - head * chunks_per_row;
    const int64_t pb = slot / bs, off = slot % bs;
    const int64_t dst = ((pb * n_kv + head) * bs + off) * chunks_per_row + cr;
    const int64_t src = ((int64_t)t * n_kv + head) * chunks_per_row + cr;
    if (blockIdx.z == 0) k_cache[dst] = k_new[src];
    else v_cache[dst] = v_new[src];
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
    const int elem = a.cache_dtype == DT_F32 ? 4 : 2;
    const int chunks_per_row = a.d_h * elem / 16;
    const int per_token = a.n_kv * chunks_per_row;
    dim3 grid((per_token + 255) / 256, a.T, 2);
    hipLaunchKernelGGL(k_append_copy, grid, dim3(256), 0, s, (const uint4*)a.k_new,
                       (const uint4*)a.v_new, a.slots, a.T, (uint4*)a.k_cache,
                       (uint4*)a.v_cache, a.n_kv, chunks_per_row, a.bs,
                       (int64_t)a.num_blocks * a.bs);
    return hipGetLastError();
}

// Quantized append: each thread encodes 16 consecutive elements of one head
// with the destination (block, head) scale and stores 16 codes (16 bytes).
// y = x * fp32(1 / scale) with an IEEE-rounded reciprocal and one rounding
// for the product, then round-to-nearest-even with saturation.
template <int SRC, int DST>
__global__ void __launch_bounds__(256) k_append_quant(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const int64_t* __restrict__ slots, int32_t T, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, int32_t n_kv, int32_t d_h, int32_t bs,
    int64_t num_slots) {
    const int32_t t = blockIdx.y;
    const int32_t groups = d_h / 16;
    const int32_t c = blockIdx.x * blockDim.x + threadIdx.x;    // over n_kv * groups
    if (t >= T || c >= n_kv * groups) return;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) return;
    const int32_t head = c / groups;
    const int32_t gi = c - head * groups;
    const int64_t pb = slot / bs, off = slot % bs;
    const bool is_v = blockIdx.z != 0;
    const float sc = (is_v ? v_scale : k_scale)[pb * n_kv + head];
    const float inv = __fdiv_rn(1.0f, sc);
    const int64_t src_elem = ((int64_t)t * n_kv + head) * d_h + gi * 16;
    float x[16];
    if (SRC == DT_F32) {
        const float4* p = (const float4*)((const float*)(is_v ? v_new : k_new) + src_elem);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 f = p[i];
            x[4 * i + 0] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
        }
    } else {
        const uint4* p = (const uint4*)((const uint16_t*)(is_v ? v_new : k_new) + src_elem);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 w = p[i];
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[8 * i + 2 * k] = bf16_lo_to_f32(ws[k]);
                x[8 * i + 2 * k + 1] = bf16_hi_to_f32(ws[k]);
            }
        }
    }
    uint32_t packed[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float y = __fmul_rn(x[4 * k + e], inv);
            uint32_t code;
            if (DST == DT_FP8) code = quant_fp8_e4m3(y);
            else code = (uint32_t)quant_int8(y) & 0xFFu;
            w |= code << (8 * e);
        }
        packed[k] = w;
    }
    const int64_t dst = ((pb * n_kv + head) * bs + off) * d_h + gi * 16;
    uint8_t* cache = is_v ? v_cache : k_cache;
    *(uint4*)(cache + dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
}

hipError_t launch_append_quant(const AppendArgs& a, hipStream_t s) {
    const int per_token = a.n_kv * (a.d_h / 16);
    dim3 grid((per_token + 255) / 256, a.T, 2);
    const int64_t num_slots = (int64_t)a.num_blocks * a.bs;
#define PDA_AQ(S, D)                                                                        \
    hipLaunchKernelGGL((k_append_quant<S, D>), grid, dim3(256), 0, s, a.k_new, a.v_new,     \
                       a.slots, a.T, (uint8_t*)a.k_cache, (uint8_t*)a.v_cache, a.k_scale,   \
                       a.v_scale, a.n_kv, a.d_h, a.bs, num_slots)
    if (a.src_dtype == DT_F32 && a.cache_dtype == DT_FP8) PDA_AQ(DT_F32, DT_FP8);
    else if (a.src_dtype == DT_F32) PDA_AQ(DT_F32, DT_INT8);
    else if (a.cache_dtype == DT_FP8) PDA_AQ(DT_BF16, DT_FP8);
    else PDA_AQ(DT_BF16, DT_INT8);
#undef PDA_AQ
    return hipGetLastError();
}

}  // namespace pda
