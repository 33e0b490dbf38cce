// merge.hip -- log-sum-exp merge of split-KV partial results.
//
// A partition's partial is (o_p, m_p, l_p): its output normalised over its own
// tokens, the max of its base-2 scores and the sum of 2^(score - m_p). Since
// softmax over the union is sum_p l_p 2^(m_p - M) o_p / sum_p l_p 2^(m_p - M)
// with M = max_p m_p, partials merge exactly; empty partials (l_p = 0) drop
// out. The split keeps the single cache read and the no-score-spill property
// of the attention step (SoK paper appendices A.1, C.4).
//
// One workgroup per output row: a block-wide max and sum over the partials'
// statistics, then S = 256 / d_h slices of the partials, each reduced over
// d_h lanes, combined through LDS.
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float v, float* red) {
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return v;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    v = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return v;
}

// context_lens != nullptr: row r belongs to sequence r / n_q and uses the
// partitions its length needs (ceil(ceil(n / 16) / bpp), capped at P);
// otherwise all P partials are read and l_p == 0 marks an empty one.
template <int HD>
__global__ void __launch_bounds__(kThreads) k_merge(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    const int32_t* __restrict__ context_lens,
                                                    int32_t n_q, int32_t P, int32_t bpp,
                                                    int32_t max_blocks, void* out,
                                                    int32_t out_dtype) {
    constexpr int S = kThreads / HD;
    __shared__ float wsh[kMaxPartitions];
    __shared__ float red[4];
    __shared__ float acc_sh[kThreads];
    const int64_t row = blockIdx.x;
    int np = P;
    bool row_bad = false;
    if (context_lens) {
        const int n = context_lens[row / n_q];
        row_bad = n < 0 || n > max_blocks * 16;
        const int nblk = row_bad ? 0 : (n + 15) >> 4;
        np = min(P, (nblk + bpp - 1) / bpp);
    }
    const float* ml = part_ml + row * (int64_t)P * 2;
    float mloc = -__builtin_inff();
    for (int p = threadIdx.x; p < np; p += kThreads) {
        const float l = ml[2 * p + 1];
        if (l != 0.0f) mloc = fmaxf(mloc, ml[2 * p]);
    }
    const float M = block_max(mloc, red);
    float lsum = 0.0f;
    for (int p = threadIdx.x; p < np; p += kThreads) {
        const float l = ml[2 * p + 1];
        const float w = l == 0.0f ? 0.0f : l * __builtin_amdgcn_exp2f(ml[2 * p] - M);
        wsh[p] = w;
        lsum += w;
    }
    const float L = block_sum(lsum, red);   // also orders the wsh writes
    const int s = threadIdx.x / HD, d = threadIdx.x % HD;
    const float* po = part_o + row * (int64_t)P * HD + d;
    float a0 = 0.0f, a1 = 0.0f;
    int p = s;
    for (; p + S < np; p += 2 * S) {
        const float w0 = wsh[p], w1 = wsh[p + S];
        if (w0 != 0.0f) a0 += w0 * po[(int64_t)p * HD];
        if (w1 != 0.0f) a1 += w1 * po[(int64_t)(p + S) * HD];
    }
    if (p < np) {
        const float w0 = wsh[p];
        if (w0 != 0.0f) a0 += w0 * po[(int64_t)p * HD];
    }
    acc_sh[threadIdx.x] = a0 + a1;
    __syncthreads();
    if (s == 0) {
        float tot = 0.0f;
#pragma unroll
        for (int k = 0; k < S; ++k) tot += acc_sh[k * HD + d];
        float r = L != 0.0f ? tot / L : 0.0f;
        if (row_bad) r = __builtin_nanf("");
        if (out_dtype == DT_F32) ((float*)out)[row * HD + d] = r;
        else ((uint16_t*)out)[row * HD + d] = (uint16_t)f32_to_bf16_rne(r);
    }
}

hipError_t launch_merge(const float* part_o, const float* part_ml, const int32_t* context_lens,
                        int32_t rows, int32_t n_q, int32_t P, int32_t bpp, int32_t max_blocks,
                        int32_t d_h, void* out, int32_t out_dtype, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    if (d_h == 128)
        hipLaunchKernelGGL((k_merge<128>), dim3(rows), dim3(kThreads), 0, s, part_o, part_ml,
                           context_lens, n_q, P, bpp, max_blocks, out, out_dtype);
    else
        hipLaunchKernelGGL((k_merge<64>), dim3(rows), dim3(kThreads), 0, s, part_o, part_ml,
                           context_lens, n_q, P, bpp, max_blocks, out, out_dtype);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_for_attn(const AttnArgs& a, hipStream_t s) {
    return launch_merge(a.part_o, a.part_ml, a.context_lens, a.B * a.n_q, a.n_q, a.P, a.bpp,
                        a.max_blocks, a.d_h, a.out, a.out_dtype, s);
}

hipError_t launch_lse_merge(const float* part_o, const float* part_ml, int32_t rows, int32_t P,
                            int32_t d_h, float* out, hipStream_t s) {
    return launch_merge(part_o, part_ml, nullptr, rows, 1, P, 1, 0, d_h, out, DT_F32, s);
}

}  // namespace pda
