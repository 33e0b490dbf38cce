// append_int4.hip -- the append path of the 4-bit cache with a residual
// window (SoK paper section 2.3: recent tokens at full precision, keys
// quantized per channel, values per token; kv-cache tag page, KV-cache
// quantization teaser).
//
// One wave per (row b, KV head j): the row's newest token (position n - 1)
// goes to residual slot (n - 1) % 16 as a bit copy; when it fills the block,
// the wave encodes the block's 16 tokens into physical block
// block_table[b][(n - 1) / 16]: lane (token tok = lane / 4, quarter qq =
// lane % 4) takes channels qq * d_h / 4 .. +d_h / 4 of token tok (token 15,
// the new one, straight from k_new / v_new; the others from the residual
// buffer, written by earlier calls) and writes their packed codes:
//   keys:   c = RNE(x * fp32(1 / k_scale[j][ch])), clamped to [-7, 7]
//   values: s = fp32(amax / 7) over the token's channels (the 4 lanes of the
//           token combine their amax; 1 if it is 0 or not finite),
//           c = RNE(x * fp32(1 / s)), clamped; v_scale[pb][j][tok] = s
// Packing: channels 8k .. 8k+7 take 4 bytes, byte i = (c[8k+i] + 8) |
// (c[8k+4+i] + 8) << 4.
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

template <int HD>
__global__ void __launch_bounds__(64) k_append_int4(const uint16_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new,
                                                    const int32_t* __restrict__ block_table,
                                                    const int32_t* __restrict__ context_lens,
                                                    uint8_t* k_q, uint8_t* v_q,
                                                    const float* __restrict__ k_scale,
                                                    float* v_scale, uint16_t* k_res,
                                                    uint16_t* v_res, int32_t n_kv,
                                                    int32_t max_blocks, int32_t num_blocks) {
    constexpr int EPL = HD / 64;   // new-row elements per lane
    constexpr int CPL = HD / 4;    // channels per lane when encoding
    constexpr int V16 = CPL / 8;   // 16-B pieces per lane when encoding
    __shared__ float kinv_sh[HD];
    const int w = blockIdx.x;
    const int b = w / n_kv, j = w - (w / n_kv) * n_kv;
    const int lane = threadIdx.x;
    const uint16_t* kn = k_new + (int64_t)w * HD;
    const uint16_t* vn = v_new + (int64_t)w * HD;
    uint16_t* kres = k_res + (int64_t)w * 16 * HD;
    uint16_t* vres = v_res + (int64_t)w * 16 * HD;
    // Every load that does not depend on the row's length is issued first,
    // together with it: the new row's elements this lane copies, the block's
    // 16 rows this lane would encode (token tok = lane / 4, channels
    // qq * CPL .. +CPL; token 15 is the new one, the others come from the
    // residual buffer) and this lane's share of the key scales.
    const int n = context_lens[b];
    uint16_t kc[EPL], vc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        kc[e] = kn[EPL * lane + e];
        vc[e] = vn[EPL * lane + e];
    }
    const int tok = lane >> 2, qq = lane & 3;
    const uint16_t* ksrc = (tok == 15 ? kn : kres + tok * HD) + qq * CPL;
    const uint16_t* vsrc = (tok == 15 ? vn : vres + tok * HD) + qq * CPL;
    uint4 kw[V16], vw[V16];
#pragma unroll
    for (int v = 0; v < V16; ++v) {
        kw[v] = *(const uint4*)(ksrc + 8 * v);
        vw[v] = *(const uint4*)(vsrc + 8 * v);
    }
    float ks_l[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) ks_l[e] = k_scale[(int64_t)j * HD + EPL * lane + e];
    if (n <= 0 || n > max_blocks * 16) return;   // uniform per wave
    const int t = n - 1, r = t & 15;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        kres[r * HD + EPL * lane + e] = kc[e];
        vres[r * HD + EPL * lane + e] = vc[e];
    }
    if (r != 15) return;
    const int pb = block_table[(int64_t)b * max_blocks + t / 16];
    // fp32(1 / k_scale) of each channel, once per wave
#pragma unroll
    for (int e = 0; e < EPL; ++e) kinv_sh[EPL * lane + e] = __fdiv_rn(1.0f, ks_l[e]);
    __syncthreads();
    float kx[CPL], vx[CPL];
#pragma unroll
    for (int v = 0; v < V16; ++v) {
        const uint32_t ka[4] = {kw[v].x, kw[v].y, kw[v].z, kw[v].w};
        const uint32_t va[4] = {vw[v].x, vw[v].y, vw[v].z, vw[v].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kx[8 * v + 2 * e] = bf16_lo_to_f32(ka[e]);
            kx[8 * v + 2 * e + 1] = bf16_hi_to_f32(ka[e]);
            vx[8 * v + 2 * e] = bf16_lo_to_f32(va[e]);
            vx[8 * v + 2 * e + 1] = bf16_hi_to_f32(va[e]);
        }
    }
    // keys, one scale per channel
    uint32_t kp[CPL / 8];
#pragma unroll
    for (int gi = 0; gi < CPL / 8; ++gi) {
        uint32_t wv = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = qq * CPL + 8 * gi + i;
            const uint32_t lo = quant_int4_nibble(__fmul_rn(kx[8 * gi + i], kinv_sh[c]));
            const uint32_t hi = quant_int4_nibble(__fmul_rn(kx[8 * gi + 4 + i], kinv_sh[c + 4]));
            wv |= (lo | (hi << 4)) << (8 * i);
        }
        kp[gi] = wv;
    }
    // values, one scale per token: amax over its channels (4 lanes)
    float amax = 0.0f;
    bool nonfinite = false;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const float v = fabsf(vx[c]);
        nonfinite = nonfinite || !(v <= 3.402823466e38f);   // NaN or infinite
        amax = fmaxf(amax, v);
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    int nf = nonfinite ? 1 : 0;
    nf |= __shfl_xor(nf, 1, 64);
    nf |= __shfl_xor(nf, 2, 64);
    const float s = (!nf && amax > 0.0f) ? __fdiv_rn(amax, 7.0f) : 1.0f;
    const float inv = __fdiv_rn(1.0f, s);
    uint32_t vp[CPL / 8];
#pragma unroll
    for (int gi = 0; gi < CPL / 8; ++gi) {
        uint32_t wv = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = quant_int4_nibble(__fmul_rn(vx[8 * gi + i], inv));
            const uint32_t hi = quant_int4_nibble(__fmul_rn(vx[8 * gi + 4 + i], inv));
            wv |= (lo | (hi << 4)) << (8 * i);
        }
        vp[gi] = wv;
    }
    if (pb < 0 || pb >= num_blocks) return;
    const int64_t row = ((int64_t)pb * n_kv + j) * 16 + tok;
    uint8_t* kd = k_q + row * (HD / 2) + qq * (CPL / 2);
    uint8_t* vd = v_q + row * (HD / 2) + qq * (CPL / 2);
    if constexpr (CPL / 8 == 4) {
        *(uint4*)kd = make_uint4(kp[0], kp[1], kp[2], kp[3]);
        *(uint4*)vd = make_uint4(vp[0], vp[1], vp[2], vp[3]);
    } else {
        *(uint2*)kd = make_uint2(kp[0], kp[1]);
        *(uint2*)vd = make_uint2(vp[0], vp[1]);
    }
    if (qq == 0) v_scale[row] = s;
}

}  // namespace

hipError_t launch_append_int4(const void* k_new, const void* v_new, const int32_t* block_table,
                              const int32_t* context_lens, void* k_q, void* v_q,
                              const float* k_scale, float* v_scale, void* k_res, void* v_res,
                              int32_t B, int32_t n_kv, int32_t d_h, int32_t max_blocks,
                              int32_t num_blocks, hipStream_t s) {
    const int64_t waves = (int64_t)B * n_kv;
    if (waves == 0) return hipSuccess;
#define PDA_AP(HD)                                                                              \
    hipLaunchKernelGGL((k_append_int4<HD>), dim3((unsigned)waves), dim3(64), 0, s,              \
                       (const uint16_t*)k_new, (const uint16_t*)v_new, block_table, context_lens, \
                       (uint8_t*)k_q, (uint8_t*)v_q, k_scale, v_scale, (uint16_t*)k_res,        \
                       (uint16_t*)v_res, n_kv, max_blocks, num_blocks)
    if (d_h == 128) PDA_AP(128);
    else PDA_AP(64);
#undef PDA_AP
    return hipGetLastError();
}

}  // namespace pda
