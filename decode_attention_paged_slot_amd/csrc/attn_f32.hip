// attn_f32.hip -- paged decode attention for fp32 caches, on the vector ALUs.
//
// Same method and the same split-KV contract as the matrix-core kernel
// (sections 9.4-9.5 of "9 Decode and KV Cache"): token t of row b is read at
// (block_table[b][t / 16], t % 16), s_t = scale * q . k_t, online softmax,
// sum of p_t v_t, over the attended positions (all, or a sliding window with
// sinks, section 9.7). Here everything stays in fp32 FMAs; this path serves fp32
// caches (small, latency-bound workloads), so it favours plainness.
//
// grid = (P partitions, n_kv, B): one workgroup (4 waves) per KV head of a
// row and partition serves all g = n_q / n_kv query heads of the group, so
// each K/V tile is read once per step (grouped-query attention: the query
// heads of a group address one stored KV head -- GQA teaser on the kv-cache
// tag page). Wave w takes head lane hg = w % HG (heads hg, hg + HG, ...) and
// block lane bl = w / HG (blocks bl, bl + BL, ... of the partition), with
// HG = min(g, 4) and BL = 4 / HG: for g >= 4 the four waves stream the same
// blocks (the tile comes from HBM once and from cache for the others), for
// g = 1 they split the blocks. In a wave, lane (t = lane / 4, part =
// lane % 4) holds token t of the block and the 16-byte column groups part,
// part + 4, ... of d_h (each load instruction reads 64 contiguous bytes of
// every row). The queries of the group wait in LDS.
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

__device__ __forceinline__ float fshfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

template <int HD, int NH>
__global__ void __launch_bounds__(kAttnThreads) k_attn_f32(AttnArgs a) {
    constexpr int NV = HD / 16;   // float4 groups per lane
    __shared__ float q_sh[4 * NH][HD];
    __shared__ float red_o[4][NH][HD];
    __shared__ float red_ml[4][NH][2];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t = lane >> 2, part = lane & 3;
    const int b = blockIdx.z, j = blockIdx.y, p = blockIdx.x;
    const int g = a.g;
    const int HG = g < 4 ? g : 4, BL = 4 / HG;
    const int hg = wave % HG, bl = wave / HG;
    const bool idle = wave >= HG * BL;   // g = 3: the fourth wave has no head lane
    const int nh = idle ? 0 : (g - hg + HG - 1) / HG;   // heads hg, hg + HG, ... < g
    const int64_t row0 = (int64_t)b * a.n_q + (int64_t)j * g;   // output row of head 0

    const int n = a.context_lens[b];
    const bool row_bad = n < 0 || n > a.max_blocks * 16;
    const int nblk = row_bad ? 0 : (n + 15) >> 4;
    const int blk0 = p * a.bpp;
    if (row_bad || blk0 >= nblk) {
        if (a.P == 1) {
            const float v = row_bad ? __builtin_nanf("") : 0.0f;
            for (int d = threadIdx.x; d < g * HD; d += kAttnThreads) {
                if (a.out_dtype == DT_F32) ((float*)a.out)[row0 * HD + d] = v;
                else ((uint16_t*)a.out)[row0 * HD + d] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
        return;
    }
    const int blk1 = (p == a.P - 1) ? nblk : min(nblk, blk0 + a.bpp);

    // the group's queries into LDS (fp32)
    for (int d = threadIdx.x; d < g * HD; d += kAttnThreads) {
        q_sh[d / HD][d % HD] = a.q_dtype == DT_F32
                                   ? ((const float*)a.q)[row0 * HD + d]
                                   : bf16_lo_to_f32(((const uint16_t*)a.q)[row0 * HD + d]);
    }
    __syncthreads();

    float m_run[NH], l_run[NH];
    float acc[NH][NV][4];
#pragma unroll
    for (int k = 0; k < NH; ++k) {
        m_run[k] = -__builtin_inff();
        l_run[k] = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[k][v][0] = acc[k][v][1] = acc[k][v][2] = acc[k][v][3] = 0.0f;
    }
    bool bad = false;
    const int64_t tile = 16 * HD;   // floats per (block, head) tile

    for (int kb = blk0 + bl; !idle && kb < blk1; kb += BL) {
        // attended positions of the block (all t < n, or the window / sinks);
        // a block without any is never looked up
        const uint32_t bm = block_token_mask(kb, n, a.window, a.sinks);
        if (bm == 0) continue;
        const int pb = a.block_table[(int64_t)b * a.max_blocks + kb];
        if (pb < 0 || pb >= a.num_blocks) { bad = true; break; }
        const bool live = (bm >> t) & 1u;
        const float* kt = (const float*)a.k + ((int64_t)pb * a.n_kv + j) * tile + t * HD;
        const float* vt = (const float*)a.v + ((int64_t)pb * a.n_kv + j) * tile + t * HD;
        // fused decode step: position n - 1 takes the new token's K/V (every
        // head of the group uses it; the waves of head lane 0 write it)
        const bool fresh = a.k_new != nullptr && 16 * kb + t == n - 1;
        const float* kn = (const float*)a.k_new + ((int64_t)b * a.n_kv + j) * HD;
        const float* vn = (const float*)a.v_new + ((int64_t)b * a.n_kv + j) * HD;
        float kv[NV][4], vv[NV][4];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float4 x = make_float4(0, 0, 0, 0), y = make_float4(0, 0, 0, 0);
            if (fresh) {
                x = *(const float4*)(kn + 4 * (part + 4 * v));
                y = *(const float4*)(vn + 4 * (part + 4 * v));
                if (hg == 0) {
                    *(float4*)(kt + 4 * (part + 4 * v)) = x;
                    *(float4*)(vt + 4 * (part + 4 * v)) = y;
                }
            } else if (live) {
                x = *(const float4*)(kt + 4 * (part + 4 * v));
                y = *(const float4*)(vt + 4 * (part + 4 * v));
            }
            kv[v][0] = x.x; kv[v][1] = x.y; kv[v][2] = x.z; kv[v][3] = x.w;
            vv[v][0] = y.x; vv[v][1] = y.y; vv[v][2] = y.z; vv[v][3] = y.w;
        }
#pragma unroll
        for (int k = 0; k < NH; ++k) {
            if (k >= nh) break;
            const float* qh = q_sh[hg + HG * k];
            float dot = 0.0f;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const float4 qv = *(const float4*)(qh + 4 * (part + 4 * v));
                dot = fmaf(qv.x, kv[v][0], dot);
                dot = fmaf(qv.y, kv[v][1], dot);
                dot = fmaf(qv.z, kv[v][2], dot);
                dot = fmaf(qv.w, kv[v][3], dot);
            }
            dot += fshfl_xor(dot, 1);
            dot += fshfl_xor(dot, 2);
            const float s = live ? dot * a.scale_log2 : -__builtin_inff();
            float mx = s;
            mx = fmaxf(mx, fshfl_xor(mx, 4));
            mx = fmaxf(mx, fshfl_xor(mx, 8));
            mx = fmaxf(mx, fshfl_xor(mx, 16));
            mx = fmaxf(mx, fshfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[k], mx);
            const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run[k] - m_use);
            const float pr = __builtin_amdgcn_exp2f(s - m_use);
            l_run[k] = l_run[k] * alpha + (part == 0 ? pr : 0.0f);
            m_run[k] = m_new;
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[k][v][e] = fmaf(pr, vv[v][e], acc[k][v][e] * alpha);
        }
    }

    // per head: reduce over the 16 token lanes (and l over all lanes), then
    // over the block lanes of the head through LDS
#pragma unroll
    for (int k = 0; k < NH; ++k) {
        if (k >= nh) break;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x = acc[k][v][e];
                x += fshfl_xor(x, 4);
                x += fshfl_xor(x, 8);
                x += fshfl_xor(x, 16);
                x += fshfl_xor(x, 32);
                acc[k][v][e] = x;
            }
        float l_tot = l_run[k];
        for (int m = 1; m < 64; m <<= 1) l_tot += fshfl_xor(l_tot, m);
        if (bad) l_tot = __builtin_nanf("");
        if (t == 0) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) red_o[wave][k][4 * (part + 4 * v) + e] = acc[k][v][e];
        }
        if (lane == 0) {
            red_ml[wave][k][0] = m_run[k];
            red_ml[wave][k][1] = l_tot;
        }
    }
    __syncthreads();
    for (int x = threadIdx.x; x < g * HD; x += kAttnThreads) {
        const int hh = x / HD, d = x - (x / HD) * HD;
        const int hl = hh % HG, k = hh / HG;   // head lane and its local head
        float M = -__builtin_inff();
        for (int q = 0; q < BL; ++q) M = fmaxf(M, red_ml[hl + HG * q][k][0]);
        float L = 0.0f, o = 0.0f;
        for (int q = 0; q < BL; ++q) {
            const int w = hl + HG * q;
            const float sc = red_ml[w][k][0] == -__builtin_inff()
                                 ? 0.0f : __builtin_amdgcn_exp2f(red_ml[w][k][0] - M);
            L += sc * red_ml[w][k][1];
            o += sc * red_o[w][k][d];
        }
        const float r = L != 0.0f ? o / L : 0.0f;
        const int64_t row = row0 + hh;
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
    dim3 grid(a.P, a.n_kv, a.B);
    // local heads per wave: ceil(g / min(g, 4))
    const int nh = a.g <= 4 ? 1 : (a.g <= 8 ? 2 : 4);
#define PDA_F32(HD, NH) hipLaunchKernelGGL((k_attn_f32<HD, NH>), grid, dim3(kAttnThreads), 0, s, a)
    if (a.d_h == 128) {
        if (nh == 1) PDA_F32(128, 1);
        else if (nh == 2) PDA_F32(128, 2);
        else PDA_F32(128, 4);
    } else {
        if (nh == 1) PDA_F32(64, 1);
        else if (nh == 2) PDA_F32(64, 2);
        else PDA_F32(64, 4);
    }
#undef PDA_F32
    return hipGetLastError();
}

}  // namespace pda
