// attn_f32.hip -- paged decode attention for fp32 caches, on the vector ALUs.
//
// Same method and the same split-KV contract as the matrix-core kernel
// (sections 9.4-9.5 of "9 Decode and KV Cache"): token t of row b is read at
// (block_table[b][t / 16], t % 16), s_t = scale * q . k_t, online softmax,
// sum of p_t v_t, over the attended positions (all, or a sliding window with
// sinks, section 9.7). Here everything stays in fp32 FMAs; this path serves fp32
// caches (small, latency-bound workloads), so it favours plainness.
//
// grid = (P partitions, n_q, B); one workgroup (4 waves) per query head and
// partition; wave w takes blocks w, w + 4, ... of the partition. In a wave,
// lane (t = lane / 4, part = lane % 4) holds token t of the block and the
// 16-byte column groups part, part + 4, ... of d_h (each load instruction
// reads 64 contiguous bytes of every row).
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

__device__ __forceinline__ float fshfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

template <int HD>
__global__ void __launch_bounds__(kAttnThreads) k_attn_f32(AttnArgs a) {
    constexpr int NV = HD / 16;   // float4 groups per lane
    __shared__ float red_o[4][HD];
    __shared__ float red_ml[4][2];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t = lane >> 2, part = lane & 3;
    const int b = blockIdx.z, h = blockIdx.y, p = blockIdx.x;
    const int j = h / a.g;
    const int64_t row = (int64_t)b * a.n_q + h;

    const int n = a.context_lens[b];
    const bool row_bad = n < 0 || n > a.max_blocks * 16;
    const int nblk = row_bad ? 0 : (n + 15) >> 4;
    const int blk0 = p * a.bpp;
    if (row_bad || blk0 >= nblk) {
        if (a.P == 1) {
            const float v = row_bad ? __builtin_nanf("") : 0.0f;
            for (int d = threadIdx.x; d < HD; d += kAttnThreads) {
                if (a.out_dtype == DT_F32) ((float*)a.out)[row * HD + d] = v;
                else ((uint16_t*)a.out)[row * HD + d] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
        return;
    }
    const int blk1 = (p == a.P - 1) ? nblk : min(nblk, blk0 + a.bpp);

    float q[NV][4];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int d = 4 * (part + 4 * k);
        if (a.q_dtype == DT_F32) {
            const float4 x = *(const float4*)((const float*)a.q + row * HD + d);
            q[k][0] = x.x; q[k][1] = x.y; q[k][2] = x.z; q[k][3] = x.w;
        } else {
            const uint2 w = *(const uint2*)((const uint16_t*)a.q + row * HD + d);
            q[k][0] = bf16_lo_to_f32(w.x); q[k][1] = bf16_hi_to_f32(w.x);
            q[k][2] = bf16_lo_to_f32(w.y); q[k][3] = bf16_hi_to_f32(w.y);
        }
    }

    float m_run = -__builtin_inff(), l_run = 0.0f;
    float acc[NV][4];
#pragma unroll
    for (int k = 0; k < NV; ++k) acc[k][0] = acc[k][1] = acc[k][2] = acc[k][3] = 0.0f;
    bool bad = false;
    const int64_t tile = 16 * HD;   // floats per (block, head) tile

    for (int kb = blk0 + wave; kb < blk1; kb += 4) {
        // attended positions of the block (all t < n, or the window / sinks);
        // a block without any is never looked up
        const uint32_t bm = block_token_mask(kb, n, a.window, a.sinks);
        if (bm == 0) continue;
        const int pb = a.block_table[(int64_t)b * a.max_blocks + kb];
        if (pb < 0 || pb >= a.num_blocks) { bad = true; break; }
        const bool live = (bm >> t) & 1u;
        const float* kt = (const float*)a.k + ((int64_t)pb * a.n_kv + j) * tile + t * HD;
        const float* vt = (const float*)a.v + ((int64_t)pb * a.n_kv + j) * tile + t * HD;
        // fused decode step: position n - 1 takes the new token's K/V (all
        // query heads of the group use it; the group's first head writes it)
        const bool fresh = a.k_new != nullptr && 16 * kb + t == n - 1;
        const float* kn = (const float*)a.k_new + ((int64_t)b * a.n_kv + j) * HD;
        const float* vn = (const float*)a.v_new + ((int64_t)b * a.n_kv + j) * HD;
        float kv[NV][4], vv[NV][4];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            float4 x = make_float4(0, 0, 0, 0), y = make_float4(0, 0, 0, 0);
            if (fresh) {
                x = *(const float4*)(kn + 4 * (part + 4 * k));
                y = *(const float4*)(vn + 4 * (part + 4 * k));
                if (h % a.g == 0) {
                    *(float4*)(kt + 4 * (part + 4 * k)) = x;
                    *(float4*)(vt + 4 * (part + 4 * k)) = y;
                }
            } else if (live) {
                x = *(const float4*)(kt + 4 * (part + 4 * k));
                y = *(const float4*)(vt + 4 * (part + 4 * k));
            }
            kv[k][0] = x.x; kv[k][1] = x.y; kv[k][2] = x.z; kv[k][3] = x.w;
            vv[k][0] = y.x; vv[k][1] = y.y; vv[k][2] = y.z; vv[k][3] = y.w;
        }
        float dot = 0.0f;
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) dot = fmaf(q[k][e], kv[k][e], dot);
        dot += fshfl_xor(dot, 1);
        dot += fshfl_xor(dot, 2);
        const float s = live ? dot * a.scale_log2 : -__builtin_inff();
        float mx = s;
        mx = fmaxf(mx, fshfl_xor(mx, 4));
        mx = fmaxf(mx, fshfl_xor(mx, 8));
        mx = fmaxf(mx, fshfl_xor(mx, 16));
        mx = fmaxf(mx, fshfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        const float pr = __builtin_amdgcn_exp2f(s - m_use);
        l_run = l_run * alpha + (part == 0 ? pr : 0.0f);
        m_run = m_new;
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[k][e] = fmaf(pr, vv[k][e], acc[k][e] * alpha);
    }

    // reduce over the 16 token lanes (and l over all lanes)
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = acc[k][e];
            v += fshfl_xor(v, 4);
            v += fshfl_xor(v, 8);
            v += fshfl_xor(v, 16);
            v += fshfl_xor(v, 32);
            acc[k][e] = v;
        }
    float l_tot = l_run;
    for (int m = 1; m < 64; m <<= 1) l_tot += fshfl_xor(l_tot, m);
    if (bad) l_tot = __builtin_nanf("");
    if (t == 0) {
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) red_o[wave][4 * (part + 4 * k) + e] = acc[k][e];
    }
    if (lane == 0) { red_ml[wave][0] = m_run; red_ml[wave][1] = l_tot; }
    __syncthreads();
    for (int d = threadIdx.x; d < HD; d += kAttnThreads) {
        float M = -__builtin_inff();
        for (int w = 0; w < 4; ++w) M = fmaxf(M, red_ml[w][0]);
        float L = 0.0f, o = 0.0f;
        for (int w = 0; w < 4; ++w) {
            const float sc = red_ml[w][0] == -__builtin_inff() ? 0.0f
                                                               : __builtin_amdgcn_exp2f(red_ml[w][0] - M);
            L += sc * red_ml[w][1];
            o += sc * red_o[w][d];
        }
        const float r = L != 0.0f ? o / L : 0.0f;
        if (a.P > 1) {
            a.part_o[(row * a.P + p) * HD + d] = r;
            if (d == 0) {
                a.part_ml[(row * a.P + p) * 2 + 0] = M;
                a.part_ml[(row * a.P + p) * 2 + 1] = L;
            }
        } else if (a.out_dtype == DT_F32) {
            ((float*)a.out)[row * HD + d] = r;
        } else {
            ((uint16_t*)a.out)[row * HD + d] = (uint16_t)f32_to_bf16_rne(r);
        }
    }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
    dim3 grid(a.P, a.n_q, a.B);
    if (a.d_h == 128) hipLaunchKernelGGL((k_attn_f32<128>), grid, dim3(kAttnThreads), 0, s, a);
    else hipLaunchKernelGGL((k_attn_f32<64>), grid, dim3(kAttnThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace pda
