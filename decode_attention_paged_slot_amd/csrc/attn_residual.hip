// attn_residual.hip -- the residual window of a 4-bit cache: each row's open
// block (its newest n % 16 tokens, held at full precision in bf16) attended
// as one split-KV piece per output row.
//
// SoK paper section 2.3: the most recent tokens stay at full precision until
// their group is quantized. The encoded blocks of the row are streamed by the
// attention kernel; this piece covers the rest, and the log-sum-exp merge
// combines the two. One wave per (row b, KV head j) takes the row's residual
// tokens t < n % 16 from k_res / v_res [B][n_kv][16][d_h] (d_h / 64 channels
// per lane) and, for each of the g query heads of the group, computes
//   s_t = scale * log2(e) * <q, k_t>   (base 2, as every piece),
//   m = max_t s_t, l = sum_t 2^(s_t - m), o = sum_t 2^(s_t - m) v_t / l,
// written to row b * n_q + j * g + hh of chunk 0 of pre_o / pre_ml. A row
// without residual tokens gets an empty piece (l = 0); an invalid row none
// (the attention kernel already wrote its NaN output). At most 15 tokens per
// row: plain vector arithmetic, no matrix cores.
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

template <int HD, int QT>
__global__ void __launch_bounds__(256) k_attn_residual(AttnArgs a) {
    constexpr int E = HD / 64;   // channels per lane
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= a.B * a.n_kv) return;   // uniform per wave
    const int b = w / a.n_kv, j = w - (w / a.n_kv) * a.n_kv;
    const int n = a.context_lens[b];
    if (n < 0 || n > a.max_blocks * 16) return;
    const int r = n % 16;
    const int g = a.g;

    float kk[16][E], vv[16][E];
    const uint16_t* kres = (const uint16_t*)a.k_res + (int64_t)w * 16 * HD + E * lane;
    const uint16_t* vres = (const uint16_t*)a.v_res + (int64_t)w * 16 * HD + E * lane;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            kk[t][e] = t < r ? __uint_as_float((uint32_t)kres[t * HD + e] << 16) : 0.0f;
            vv[t][e] = t < r ? __uint_as_float((uint32_t)vres[t * HD + e] << 16) : 0.0f;
        }
    }
    for (int hh = 0; hh < g; ++hh) {
        const int64_t row = (int64_t)b * a.n_q + j * g + hh;
        if (r == 0) {
            if (lane == 0) *(float2*)(a.pre_ml + row * 2) = make_float2(-__builtin_inff(), 0.0f);
            continue;
        }
        float q[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int64_t qi = row * HD + E * lane + e;
            q[e] = QT == DT_BF16 ? __uint_as_float((uint32_t)((const uint16_t*)a.q)[qi] << 16)
                                 : ((const float*)a.q)[qi];
        }
        float s[16];
        float m = -__builtin_inff();
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float p = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) p += q[e] * kk[t][e];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) p += __shfl_xor(p, o, 64);
            s[t] = t < r ? p * a.scale_log2 : -__builtin_inff();
            m = fmaxf(m, s[t]);
        }
        float l = 0.0f, acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const float wt = t < r ? __builtin_amdgcn_exp2f(s[t] - m) : 0.0f;
            l += wt;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += wt * vv[t][e];
        }
        const float inv = 1.0f / l;
#pragma unroll
        for (int e = 0; e < E; ++e) a.pre_o[row * HD + E * lane + e] = acc[e] * inv;
        if (lane == 0) *(float2*)(a.pre_ml + row * 2) = make_float2(m, l);
    }
}

}  // namespace

hipError_t launch_attn_residual(const AttnArgs& a, hipStream_t s) {
    const int64_t waves = (int64_t)a.B * a.n_kv;
    if (waves == 0) return hipSuccess;
    const dim3 grid((unsigned)((waves + 3) / 4));
#define PDA_RES(HD, QT) hipLaunchKernelGGL((k_attn_residual<HD, QT>), grid, dim3(256), 0, s, a)
    if (a.d_h == 128) {
        if (a.q_dtype == DT_BF16) PDA_RES(128, DT_BF16);
        else PDA_RES(128, DT_F32);
    } else {
        if (a.q_dtype == DT_BF16) PDA_RES(64, DT_BF16);
        else PDA_RES(64, DT_F32);
    }
#undef PDA_RES
    return hipGetLastError();
}

}  // namespace pda
