// attn_residual.hip -- the residual window of a 4-bit cache: each row's open
// block (its newest n % 16 tokens, held at full precision in bf16) attended
// as one split-KV piece per output row.
//
// SoK paper section 2.3: the most recent tokens stay at full precision until
// their group is quantized. The encoded blocks of the row are streamed by the
// attention kernel; this piece covers the rest, and the log-sum-exp merge
// combines the two. One wave per output row (b, h), j = h / g: lane
// (token t = lane / 4, quarter qq = lane % 4) forms the partial dot product
// of q with k_t over channels qq * d_h / 4 .. +d_h / 4, so the 16 scores
//   s_t = scale * log2(e) * <q, k_t>   (base 2, as every piece)
// come out together after two shuffles; then m = max_t s_t,
// l = sum_t 2^(s_t - m) and lane L sums o = sum_t 2^(s_t - m) v_t / l over its
// d_h / 64 channels. The piece goes to row b * n_q + h of chunk 0 of
// pre_o / pre_ml. A row without residual tokens gets an empty piece (l = 0);
// an invalid row none (the attention kernel already wrote its NaN output).
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

template <int HD, int QT>
__global__ void __launch_bounds__(256) k_attn_residual(AttnArgs a) {
    constexpr int CQ = HD / 4;    // channels per lane in the score phase
    constexpr int E = HD / 64;    // channels per lane in the output phase
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // b * n_q + h
    if (row >= (int64_t)a.B * a.n_q) return;   // uniform per wave
    const int b = (int)(row / a.n_q), h = (int)(row - (int64_t)b * a.n_q);
    const int j = h / a.g;
    const int n = a.context_lens[b];
    if (n < 0 || n > a.max_blocks * 16) return;
    const int r = n % 16;
    if (r == 0) {
        if (lane == 0) *(float2*)(a.pre_ml + row * 2) = make_float2(-__builtin_inff(), 0.0f);
        return;
    }
    const int64_t base = ((int64_t)b * a.n_kv + j) * 16 * HD;   // residual rows of (b, j)
    const int t = lane >> 2, qq = lane & 3;
    // scores: lane (t, qq) over channels qq * CQ .. +CQ
    float p = 0.0f;
    if (t < r) {
        const uint16_t* kp = (const uint16_t*)a.k_res + base + t * HD + qq * CQ;
#pragma unroll
        for (int c = 0; c < CQ; c += 8) {
            const uint4 kw = *(const uint4*)(kp + c);
            const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w};
            float qv[8];
            if (QT == DT_BF16) {
                const uint4 qw = *(const uint4*)((const uint16_t*)a.q + row * HD + qq * CQ + c);
                const uint32_t qs[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    qv[2 * k] = bf16_lo_to_f32(qs[k]);
                    qv[2 * k + 1] = bf16_hi_to_f32(qs[k]);
                }
            } else {
                const float* qf = (const float*)a.q + row * HD + qq * CQ + c;
#pragma unroll
                for (int k = 0; k < 8; ++k) qv[k] = qf[k];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                p += qv[2 * k] * bf16_lo_to_f32(kk[k]) + qv[2 * k + 1] * bf16_hi_to_f32(kk[k]);
        }
    }
    p += __shfl_xor(p, 1, 64);
    p += __shfl_xor(p, 2, 64);
    const float s = t < r ? p * a.scale_log2 : -__builtin_inff();
    float m = s;
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float w = t < r ? __builtin_amdgcn_exp2f(s - m) : 0.0f;
    float l = qq == 0 ? w : 0.0f;   // one lane per token, summed over all lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) l += __shfl_xor(l, o, 64);
    // output: lane L over channels E * L .. +E
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    const uint16_t* vp = (const uint16_t*)a.v_res + base + E * lane;
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
        const float wt = __shfl(w, 4 * tt, 64);
        if (tt < r) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[e] += wt * __uint_as_float((uint32_t)vp[tt * HD + e] << 16);
        }
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < E; ++e) a.pre_o[row * HD + E * lane + e] = acc[e] * inv;
    if (lane == 0) *(float2*)(a.pre_ml + row * 2) = make_float2(m, l);
}

}  // namespace

hipError_t launch_attn_residual(const AttnArgs& a, hipStream_t s) {
    const int64_t waves = (int64_t)a.B * a.n_q;   // one per output row
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
