// attn_prefix.hip -- the shared-prefix pass of paged decode attention: each
// block of a prompt prefix that many rows share is read from memory once and
// applied to the queries of every row that starts with it.
//
// What is computed (SoK paper section 2.6: prefix sharing stores a prefix's
// KV state once for all requests that share it; the attention itself as in
// sections 9.4-9.5 of "9 Decode and KV Cache"): for KV head j, a chunk of
// kPrefixChunk consecutive prefix blocks, and every query head h = j * g + hh
// of every row b whose shared prefix (prefix_lens[b] blocks) reaches into the
// chunk, the softmax of scale * <q[b][h], K_t> restricted to the chunk's
// positions inside row b's prefix, applied to V_t. The result is a partial
// in the split-KV form (normalised output, base-2 max, sum) that the
// log-sum-exp merge combines with the row's other pieces; the prefix blocks
// are complete (copy on write keeps the block of a row's newest position
// private), so every position of a prefix block is attended.
//
// Work decomposition. A workgroup takes (KV head, chunk, query group of 64
// queries); query qi = b * g + hh of head group j is output row
// b * n_q + j * g + hh. It issues its query loads, reads the chunk's block
// ids into LDS, then issues the loads of all of the chunk's K and V tiles
// and of the blocks' scales at once (one memory round trip) and writes them
// to LDS, the tiles as bf16
// (8-bit caches are converted here, once per workgroup). Eight waves share
// the tiles: wave w owns the 16 queries of tile w % 4 (the N columns of its
// matrix products) over the chunk's blocks of parity w / 4, two blocks per
// online-softmax step, so two waves per SIMD and two independent score
// products per wave hide each other's latency:
//   S^T[16 tok][16 q] = K_tile . Q^T            -- MFMA 16x16x32 bf16
//   O^T[d_h][16 q] += [V^T | V^T] . [P_hi; P_lo] -- MFMA 16x16x32 bf16
// with the same lazy online softmax as the streaming kernel; the two parities'
// partial softmaxes are merged through LDS before the one write. The query
// groups of one (head, chunk) run on the same XCD, so their repeated reads of
// the chunk's tiles hit that XCD's L2.
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

constexpr float kSlack = 8.0f;   // lazy-rescaling threshold (weights < 2^8)

constexpr int kPrefixThreads = 512;   // 8 waves: 4 query tiles x 2 block parities

template <int HD, int KV, int QT>
__global__ void __launch_bounds__(kPrefixThreads) k_attn_prefix(AttnArgs a, int32_t units,
                                                                int32_t qgroups) {
    constexpr bool QUANT = KV != DT_BF16;
    constexpr int W = QUANT ? 1 : 2;                   // bytes per cached element
    constexpr int ROWB = HD * W;                       // bytes per cached token row
    constexpr int TILEB = 16 * ROWB;                   // bytes per (block, head) tile
    constexpr int HALF = TILEB / 16;                   // 16-B chunks per tile
    constexpr int CH = 2 * HALF;                       // 16-B chunks of a block's K and V
    constexpr int LPT = (kPrefixChunk * CH + kPrefixThreads - 1) / kPrefixThreads;
    constexpr int LROW = HD * 2;                       // bytes per bf16 LDS row
    constexpr int LTILE = 16 * LROW;
    constexpr int NCH = HD / 32;                       // QK k-chunks
    constexpr int NT = HD / 16;                        // PV output tiles
    __shared__ __attribute__((aligned(16))) char kl[kPrefixChunk * LTILE];
    __shared__ __attribute__((aligned(16))) char vl[kPrefixChunk * LTILE];
    __shared__ float ksl[kPrefixChunk], vsl[kPrefixChunk];
    __shared__ int idl[kPrefixChunk];
    __shared__ int wneed[8];

    // workgroup -> (unit = (chunk, KV head), query group); the query groups
    // of a unit share blockIdx.x % 8, i.e. one XCD
    const int L = blockIdx.x;
    const int xcd = L & 7, rest = L >> 3;
    const int qg = rest % qgroups;
    const int u = (rest / qgroups) * 8 + xcd;
    if (u >= units) return;   // grid padding (uniform per workgroup)
    const int n_kv = a.n_kv, g = a.g;
    const int chunk = u / n_kv, j = u - (u / n_kv) * n_kv;
    const int i0 = chunk * kPrefixChunk;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qt = wave & 3;     // query tile of the workgroup's 64 queries
    const int par = wave >> 2;   // this wave takes the chunk's blocks of this parity
    const int col = lane & 15;   // token row (A operand) / query (B, D)
    const int grp = lane >> 4;

    // this lane's query (column `col` of its wave's tile) and its prefix
    const int Bg = a.B * g;
    const int qi = qg * 64 + qt * 16 + col;
    int pq = 0;
    int64_t orow = 0;
    if (qi < Bg) {
        const int b = qi / g, hh = qi - (qi / g) * g;
        pq = max(row_prefix_len(a.context_lens[b], a.prefix_lens[b], a.max_blocks,
                                a.prefix_blocks), 0);
        orow = (int64_t)b * a.n_q + j * g + hh;
    }
    const bool live = pq > i0;                         // its prefix reaches into the chunk
    // query operands (B operand of S^T = K . Q^T), issued first so their
    // latency overlaps the tile loads: lane (query col, grp) holds elements
    // 32 c + 8 grp .. +7 of its query
    bf16x8 qhi[NCH], qlo[NCH];
    {
        const bool ql = qi < Bg;
        const int64_t qrow = ql ? orow * HD : 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int d0 = 32 * c + 8 * grp;
            if (QT == DT_BF16) {
                uint4 w = make_uint4(0, 0, 0, 0);
                if (ql) w = *(const uint4*)((const char*)a.q + (qrow + d0) * 2);
                qhi[c] = __builtin_bit_cast(bf16x8, w);
            } else {
                float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (ql) {
                    const float4 x0 = *(const float4*)((const float*)a.q + qrow + d0);
                    const float4 x1 = *(const float4*)((const float*)a.q + qrow + d0 + 4);
                    f[0] = x0.x; f[1] = x0.y; f[2] = x0.z; f[3] = x0.w;
                    f[4] = x1.x; f[5] = x1.y; f[6] = x1.z; f[7] = x1.w;
                }
                uint32_t h16[8], l16[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) split_bf16(f[e], h16[e], l16[e]);
                u32x4 hv = {h16[0] | (h16[1] << 16), h16[2] | (h16[3] << 16),
                            h16[4] | (h16[5] << 16), h16[6] | (h16[7] << 16)};
                u32x4 lv = {l16[0] | (l16[1] << 16), l16[2] | (l16[3] << 16),
                            l16[4] | (l16[5] << 16), l16[6] | (l16[7] << 16)};
                qhi[c] = __builtin_bit_cast(bf16x8, hv);
                qlo[c] = __builtin_bit_cast(bf16x8, lv);
            }
        }
    }
    const int mylen = live ? min(pq - i0, kPrefixChunk) : 0;   // chunk blocks it attends
    int wn = mylen;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) wn = max(wn, __shfl_xor(wn, m, 64));
    wn = __builtin_amdgcn_readfirstlane(wn);
    if (lane == 0) wneed[wave] = wn;
    // the chunk's block ids (one lane per block); an unmapped entry is read
    // as block 0 and its tiles zeroed, its rows poisoned below
    int sid = -1;   // this lane's block id, for its block's scales
    if ((int)threadIdx.x < kPrefixChunk) {
        const int blk = threadIdx.x;
        int id = blk < a.prefix_blocks - i0 ? a.prefix_table[i0 + blk] : 0;
        const bool ok = id >= 0 && id < a.num_blocks;
        idl[blk] = ok ? id : -1;
        sid = ok ? id : -1;
    }
    __syncthreads();
    int nb = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) nb = max(nb, wneed[w]);
    if (nb == 0) return;   // no row of this query group shares the chunk (uniform)

    // all of the chunk's K and V tiles in flight at once, unconditionally
    const int64_t head_off = (int64_t)j * TILEB;
    const int64_t block_stride = (int64_t)n_kv * TILEB;
    uint4 raw[LPT];
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
        const int idx = threadIdx.x + kPrefixThreads * l;
        const int blk = min(idx / CH, nb - 1), ch = idx - (idx / CH) * CH;
        const int id = max(idl[blk], 0);
        const char* base = (ch < HALF ? (const char*)a.k : (const char*)a.v) +
                           (int64_t)id * block_stride + head_off + 16 * (ch % HALF);
        raw[l] = *(const uint4*)base;
    }
    // the block scales, requested after the tiles so that the two share a
    // round trip (the loop reads them after the barrier below)
    if constexpr (QUANT) {
        if ((int)threadIdx.x < kPrefixChunk) {
            ksl[threadIdx.x] = sid >= 0 ? a.k_scale[(int64_t)sid * n_kv + j] : 0.0f;
            vsl[threadIdx.x] = sid >= 0 ? a.v_scale[(int64_t)sid * n_kv + j] : 0.0f;
        }
    } else {
        (void)sid;
    }
    // to LDS as bf16: K rows with the chunk XOR swizzle of the operand read,
    // V rows in the layout of the transposed reads
#pragma unroll
    for (int l = 0; l < LPT; ++l) {
        const int idx = threadIdx.x + kPrefixThreads * l;
        const int blk = idx / CH, ch = idx - (idx / CH) * CH;
        if (blk < nb) {
            const uint4 w = idl[blk] < 0 ? make_uint4(0, 0, 0, 0) : raw[l];
            const bool isk = ch < HALF;
            const int byte = 16 * (ch % HALF);
            const int r = byte / ROWB;
            const int cb = ((byte % ROWB) / W) / 8;   // bf16 chunk of the first element
            char* tile = (isk ? kl : vl) + blk * LTILE;
            if constexpr (!QUANT) {
                if (isk) *(uint4*)(tile + r * LROW + 16 * (cb ^ kswz<HD>(r))) = w;
                else *(uint4*)(tile + lds_off<HD>(r, cb)) = w;
            } else {
                const bf16x8 x0 = kv_operand_from_bytes<KV>(w, 0);
                const bf16x8 x1 = kv_operand_from_bytes<KV>(w, 1);
                if (isk) {
                    *(bf16x8*)(tile + r * LROW + 16 * (cb ^ kswz<HD>(r))) = x0;
                    *(bf16x8*)(tile + r * LROW + 16 * ((cb + 1) ^ kswz<HD>(r))) = x1;
                } else {
                    *(bf16x8*)(tile + lds_off<HD>(r, cb)) = x0;
                    *(bf16x8*)(tile + lds_off<HD>(r, cb + 1)) = x1;
                }
            }
        }
    }
    __syncthreads();

    // transposed-read offsets of the value operand, as in the streaming kernel
    int trd0[NT], trd1[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int base = (grp & 1) * 8, q4 = lane & 3;
        const int r0 = base + ((lane & 15) >> 2);
        trd0[t] = lds_off<HD>(r0, 2 * t + (q4 >> 1)) + 8 * (q4 & 1);
        trd1[t] = lds_off<HD>(r0 + 4, 2 * t + (q4 >> 1)) + 8 * (q4 & 1);
    }

    float m_run = -__builtin_inff();
    float l_run = 0.0f;
    bool bad = false;
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};

    auto scores = [&](int blk) {
        const char* kt = kl + blk * LTILE;
        f32x4 st = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const bf16x8 kop =
                *(const bf16x8*)(kt + col * LROW + 16 * ((4 * c + grp) ^ kswz<HD>(col)));
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qhi[c], st, 0, 0, 0);
            if (QT == DT_F32) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qlo[c], st, 0, 0, 0);
        }
        return st;
    };
    // P split into bf16 hi + lo and regrouped into the packed B operand
    auto p_operand = [&](const float* pe, float vsc) {
        uint32_t H[2], Lw[2];
        split_bf16x2(pe[0] * vsc, pe[1] * vsc, H[0], Lw[0]);
        split_bf16x2(pe[2] * vsc, pe[3] * vsc, H[1], Lw[1]);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto x = __builtin_amdgcn_permlane32_swap(H[w], Lw[w], false, false);
            const auto y = __builtin_amdgcn_permlane16_swap(x[0], x[1], false, false);
            H[w] = y[0];
            Lw[w] = y[1];
        }
        const u32x4 pb4 = {H[0], H[1], Lw[0], Lw[1]};
        return __builtin_bit_cast(bf16x8, pb4);
    };
    auto pv = [&](int blk, bf16x8 pop) {
        const char* vt = vl + blk * LTILE;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(vt + trd0[t]));
            const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(vt + trd1[t]));
            const s16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pop,
                                                              acc[t], 0, 0, 0);
        }
    };

    // blocks b0 and b0 + 2 of this wave's parity per step, one online-softmax
    // update over their 32 tokens (two independent score products in flight)
    for (int b0 = par; b0 < wn; b0 += 4) {   // wn is wave-uniform
        const int b1 = b0 + 2;
        const bool two = b1 < wn;            // wave-uniform
        const f32x4 st0 = scores(b0);
        const f32x4 st1 = two ? scores(b1) : f32x4{0, 0, 0, 0};
        const bool on0 = b0 < mylen;         // the block is in this query's prefix
        const bool on1 = two && b1 < mylen;
        if ((on0 && idl[b0] < 0) || (on1 && idl[b1] < 0)) bad = true;
        const float mult0 = a.scale_log2 * (QUANT ? ksl[b0] : 1.0f);
        const float mult1 = two ? a.scale_log2 * (QUANT ? ksl[b1] : 1.0f) : 0.0f;
        float sv0[4], sv1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sv0[e] = on0 ? st0[e] * mult0 : -__builtin_inff();
            sv1[e] = on1 ? st1[e] * mult1 : -__builtin_inff();
        }
        const float mx = max_rows4(fmaxf(fmaxf(fmaxf(sv0[0], sv0[1]), fmaxf(sv0[2], sv0[3])),
                                         fmaxf(fmaxf(sv1[0], sv1[1]), fmaxf(sv1[2], sv1[3]))));
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
            const float m_new = mx > m_run + kSlack ? mx : m_run;
            const float alpha = m_run == -__builtin_inff() ? 0.0f
                                                           : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -__builtin_inff() ? 0.0f : m_run;
        float pe0[4], pe1[4], psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pe0[e] = __builtin_amdgcn_exp2f(sv0[e] - m_use);
            pe1[e] = __builtin_amdgcn_exp2f(sv1[e] - m_use);
            psum += pe0[e] + pe1[e];
        }
        l_run += psum;
        pv(b0, p_operand(pe0, QUANT ? vsl[b0] : 1.0f));
        if (two) pv(b1, p_operand(pe1, QUANT ? vsl[b1] : 1.0f));
    }

    // the odd-block waves hand their state to the even-block waves of the
    // same query tile through LDS (the K tiles are no longer read); the two
    // partial softmaxes merge exactly: M = max, weights 2^(m - M)
    __syncthreads();
    float* xs = (float*)kl + (size_t)(qt * 64 + lane) * (NT * 4 + 3);
    if (par == 1) {
        xs[0] = m_run;
        xs[1] = l_run;
        xs[2] = bad ? 1.0f : 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[3 + 4 * t + e] = acc[t][e];
    }
    __syncthreads();
    if (par == 1) return;
    {
        const float m1 = xs[0];
        const float M = fmaxf(m_run, m1);
        const float a0 = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
        const float a1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
        l_run = l_run * a0 + xs[1] * a1;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t][e] = acc[t][e] * a0 + xs[3 + 4 * t + e] * a1;
        m_run = M;
        bad = bad || xs[2] != 0.0f;
    }

    // the piece of each live query: row chunk * rows + orow of pre_o / pre_ml
    float l_tot = sum_rows4(l_run);
    if (bad) l_tot = __builtin_nanf("");
    if (live) {
        const int64_t prow = (int64_t)chunk * ((int64_t)a.B * a.n_q) + orow;
        const float inv = l_tot != 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            *(f32x4*)(a.pre_o + prow * HD + 16 * t + 4 * grp) = acc[t] * inv;
        if (grp == 0) *(float2*)(a.pre_ml + prow * 2) = make_float2(m_run, l_tot);
    }
}

}  // namespace

hipError_t launch_attn_prefix(const AttnArgs& a, hipStream_t s) {
    if (a.B == 0 || a.prefix_blocks <= 0) return hipSuccess;
    const int32_t chunks = (a.prefix_blocks + kPrefixChunk - 1) / kPrefixChunk;
    const int32_t units = chunks * a.n_kv;
    const int32_t qgroups = (int32_t)(((int64_t)a.B * a.g + 63) / 64);
    const int64_t wgs = (int64_t)((units + 7) / 8) * 8 * qgroups;
    dim3 grid((unsigned)wgs);
    dim3 block(kPrefixThreads);
#define PDA_LAUNCH(HD, KV, QT) \
    hipLaunchKernelGGL((k_attn_prefix<HD, KV, QT>), grid, block, 0, s, a, units, qgroups)
#define PDA_BY_Q(HD, KV)                                   \
    if (a.q_dtype == DT_BF16) PDA_LAUNCH(HD, KV, DT_BF16); \
    else PDA_LAUNCH(HD, KV, DT_F32)
#define PDA_BY_KV(HD)                                         \
    if (a.kv_dtype == DT_BF16) { PDA_BY_Q(HD, DT_BF16); }     \
    else if (a.kv_dtype == DT_FP8) { PDA_BY_Q(HD, DT_FP8); }  \
    else { PDA_BY_Q(HD, DT_INT8); }
    if (a.d_h == 128) { PDA_BY_KV(128); }
    else { PDA_BY_KV(64); }
#undef PDA_BY_KV
#undef PDA_BY_Q
#undef PDA_LAUNCH
    return hipGetLastError();
}

}  // namespace pda
