// attn_mfma.hip -- paged single-token decode attention on CDNA4 matrix cores,
// for 16-bit (bf16) and 8-bit (fp8 e4m3 / int8 + per-block scale) caches.
//
// What is computed (sections 9.4-9.5 of "9 Decode and KV Cache"; SoK paper
// section 1.1): for every sequence b, KV head j and the g = n_q / n_kv query
// heads h of its group, softmax(scale * q_h . K_t) over t < n_b, applied to
// V_t, where token t lives at (block_table[b][t / 16], t % 16). One read of
// each (block, head) K/V tile serves all g query heads (the GQA reuse that
// gives 2 g / w_kv FLOP per byte), scores never leave registers.
//
// Work decomposition (one workgroup = 4 waves = 256 lanes):
//   grid = (P partitions, n_kv, B). Partition p of row b owns the contiguous
//   logical blocks [p * bpp, (p + 1) * bpp) (the last partition runs to the end
//   of the row); wave w of the workgroup takes blocks w, w + 4, w + 8, ... of
//   it, each wave with its own online-softmax state; the four states are
//   merged through LDS at the end. With P > 1 the workgroup writes a partial
//   (normalised output, max, sum) and a log-sum-exp merge kernel finishes.
//
// Per 16-token block and wave:
//   S^T[16 tok][16 heads] = K_tile[16][d_h] . Q^T[d_h][16]  -- MFMA 16x16x32 bf16;
//     K goes from HBM straight into the A-operand registers: lane (t, grp)
//     loads 16 contiguous bytes of token row t, so each load instruction
//     covers 16 rows x 64 contiguous bytes; Q sits in the B operand with the
//     same element order (the contraction order over d_h is free).
//   The S^T accumulator layout puts 4 tokens of one head in each lane, which
//   is exactly the B-operand layout of the value product, so the
//   probabilities never move between lanes.
//   O^T[d_h][16 heads] += V^T[d_h][16 tok] . P^T[16 tok][16]  -- MFMA 16x16x16
//     bf16; V is staged through LDS (XOR-swizzled rows, conflict-free) and
//     read back transposed with ds_read_b64_tr_b16. P is split into bf16
//     hi + lo parts (two MFMAs) so the weights keep ~16 bits; Q in fp32 is
//     split the same way.
//   8-bit caches are converted to bf16 in registers (exact), the K scale is
//   folded into the score multiplier and the V scale into P.
// Loads run `kDepth` blocks ahead of the math in each wave.
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

constexpr int kDepth = 2;   // blocks in flight per wave beyond the one being consumed

template <int HD, int KV>
struct Tr {
    static constexpr int W = (KV == DT_BF16) ? 2 : 1;   // bytes per cached element
    static constexpr int ROWB = HD * W;                 // bytes per token row
    static constexpr int TILEB = 16 * ROWB;             // bytes per (block, head) tile
    static constexpr int LOADS = TILEB / 1024;          // 16-B loads per lane per tile
    static constexpr int NCH = HD / 32;                 // QK k-chunks
    static constexpr int NT = HD / 16;                  // PV output tiles
    static constexpr int LROW = HD * 2;                 // bytes per bf16 LDS row
    static constexpr int LTILE = 16 * LROW;
    static constexpr int CPR = HD / 8;                  // 16-B chunks per LDS row
    static constexpr int RPS = 256 / LROW;              // LDS rows per 256 B
};

// First element of QK chunk c held by lane group grp (8 consecutive elements).
template <int HD, int KV>
__device__ __forceinline__ constexpr int dmap(int c, int grp) {
    return KV == DT_BF16 ? 32 * c + 8 * grp : 64 * (c / 2) + 16 * grp + 8 * (c % 2);
}

// Byte offset of (row t, 16-B chunk cb) in a bf16 LDS tile; the XOR keeps the
// 16 rows of a transposed read on distinct banks.
template <int HD>
__device__ __forceinline__ int lds_off(int t, int cb) {
    constexpr int CPR = HD / 8, RPS = 256 / (HD * 2);
    const int f = 2 * ((t / RPS) % (CPR / 2));
    return t * (HD * 2) + 16 * (cb ^ f);
}

__device__ __forceinline__ uint4 ld16(const char* p) { return *(const uint4*)p; }

// Streaming 16-B load of cache data: every K/V byte is read exactly once per
// step, so the load is marked non-temporal and does not displace reusable
// lines (block table, queries) from the caches.
__device__ __forceinline__ uint4 ld16_stream(const char* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float fshfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

template <int KV>
__device__ __forceinline__ bf16x8 kv_operand_from_bytes(uint4 w, int half) {
    if (KV == DT_BF16) {
        return __builtin_bit_cast(bf16x8, w);
    } else {
        const uint32_t a = half ? w.z : w.x;
        const uint32_t b = half ? w.w : w.y;
        u32x2 lo, hi;
        if (KV == DT_FP8) { lo = fp8x4_to_bf16x4(a); hi = fp8x4_to_bf16x4(b); }
        else { lo = int8x4_to_bf16x4(a); hi = int8x4_to_bf16x4(b); }
        u32x4 r = {lo.x, lo.y, hi.x, hi.y};
        return __builtin_bit_cast(bf16x8, r);
    }
}

template <int HD, int KV, int QT>
__global__ void __launch_bounds__(kAttnThreads, 2) k_attn_mfma(AttnArgs a) {
    using T = Tr<HD, KV>;
    constexpr bool QUANT = KV != DT_BF16;
    constexpr int OROW = HD + 4;   // padded fp32 row of the combine buffer
    constexpr int STAGE_BYTES = 4 * T::LTILE;
    constexpr int COMB_BYTES = 4 * 16 * OROW * 4 + 4 * 16 * 2 * 4;
    constexpr int SMEM = STAGE_BYTES > COMB_BYTES ? STAGE_BYTES : COMB_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int col = lane & 15;   // token row (A operand) / query head (B, D)
    const int grp = lane >> 4;
    const int b = blockIdx.z, j = blockIdx.y, p = blockIdx.x;
    const int g = a.g;

    const int n = a.context_lens[b];
    const bool row_bad = n < 0 || n > a.max_blocks * 16;
    const int nblk = row_bad ? 0 : (n + 15) >> 4;
    const int blk0 = p * a.bpp;
    if (row_bad || blk0 >= nblk) {
        // unsplit: this workgroup owns the row's output (NaN for a bad row,
        // zeros for an empty one); split: the merge kernel handles the row
        if (a.P == 1) {
            const float v = row_bad ? __builtin_nanf("") : 0.0f;
            for (int idx = threadIdx.x; idx < g * HD; idx += kAttnThreads) {
                const int h = idx / HD, d = idx % HD;
                const int64_t o = ((int64_t)b * a.n_q + j * g + h) * HD + d;
                if (a.out_dtype == DT_F32) ((float*)a.out)[o] = v;
                else ((uint16_t*)a.out)[o] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
        return;
    }
    const int blk1 = (p == a.P - 1) ? nblk : min(nblk, blk0 + a.bpp);
    const int nb_wg = blk1 - blk0;
    const int my_cnt = nb_wg > wave ? (nb_wg - wave + 3) >> 2 : 0;

    // ---- query operands (B operand of S^T = K . Q^T): lane (h, grp)
    bf16x8 qhi[T::NCH], qlo[T::NCH];
    {
        const bool live = col < g;
        const int64_t qrow = ((int64_t)b * a.n_q + j * g + (live ? col : 0)) * HD;
#pragma unroll
        for (int c = 0; c < T::NCH; ++c) {
            const int d0 = dmap<HD, KV>(c, grp);
            if (QT == DT_BF16) {
                uint4 w = make_uint4(0, 0, 0, 0);
                if (live) w = ld16((const char*)a.q + (qrow + d0) * 2);
                qhi[c] = __builtin_bit_cast(bf16x8, w);
            } else {
                float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (live) {
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

    // ---- per-wave state
    float m_run = -__builtin_inff();
    float l_run = 0.0f;
    f32x4 acc[T::NT];
#pragma unroll
    for (int t = 0; t < T::NT; ++t) acc[t] = f32x4{0, 0, 0, 0};
    bool bad = false;

    char* stage = smem + wave * T::LTILE;
    const char* kbase = (const char*)a.k;
    const char* vbase = (const char*)a.v;
    const int64_t head_stride = T::TILEB;
    const int64_t block_stride = (int64_t)a.n_kv * T::TILEB;

    // V row / chunk handled by this lane for load l of a tile
    int vrow[T::LOADS], vcb[T::LOADS];
#pragma unroll
    for (int l = 0; l < T::LOADS; ++l) {
        const int byte = 1024 * l + 16 * lane;
        vrow[l] = byte / T::ROWB;
        vcb[l] = ((byte % T::ROWB) / T::W) / 8;   // bf16 chunk of the first element
    }
    // transposed-read addresses for the value operand: lane L reads row L/4,
    // columns 16 n + 4 (L % 4) .. +3
    int trd[T::NT];
#pragma unroll
    for (int t = 0; t < T::NT; ++t) {
        const int r = lane >> 2, q4 = lane & 3;
        trd[t] = lds_off<HD>(r, 2 * t + (q4 >> 1)) + 8 * (q4 & 1);
    }

    for (int base = 0; base < my_cnt && !bad; base += 64) {
        const int cnt = min(64, my_cnt - base);
        // lane i holds the physical block (and scales) of this wave's i-th block
        int id = 0;
        float ksc = 1.0f, vsc = 1.0f;
        const int kb_lane = blk0 + wave + 4 * (base + lane);
        if (lane < cnt) {
            id = a.block_table[(int64_t)b * a.max_blocks + kb_lane];
            if (QUANT && id >= 0 && id < a.num_blocks) {
                ksc = a.k_scale[(int64_t)id * a.n_kv + j];
                vsc = a.v_scale[(int64_t)id * a.n_kv + j];
            }
        }
        if (__ballot(lane < cnt && (id < 0 || id >= a.num_blocks)) != 0) {
            bad = true;
            break;
        }

        uint4 kr[kDepth][T::LOADS], vr[kDepth][T::LOADS];

        // Loads are never predicated (a partially filled final block is still a
        // whole allocated tile; its tail rows are masked after loading), so
        // every refill issues the same instructions and the waits before each
        // block's math only drain that block's loads.
        auto issue = [&](int s, int i) {
            const int pb = __builtin_amdgcn_readlane(id, i);
            const char* kt = kbase + (int64_t)pb * block_stride + (int64_t)j * head_stride;
            const char* vt = vbase + (int64_t)pb * block_stride + (int64_t)j * head_stride;
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l) kr[s][l] = ld16_stream(kt + col * T::ROWB + 64 * l + 16 * grp);
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l) vr[s][l] = ld16_stream(vt + 1024 * l + 16 * lane);
        };

        auto consume = [&](int s, int i, bool refill) {
            const int kb = blk0 + wave + 4 * (base + i);
            const int valid = min(16, n - 16 * kb);
            if (valid < 16) {
                // rows past the row's end hold stale data (possibly NaN):
                // zero them so that 0-weight products stay 0
#pragma unroll
                for (int l = 0; l < T::LOADS; ++l)
                    if (vrow[l] >= valid) vr[s][l] = make_uint4(0, 0, 0, 0);
            }
            // stage V (as bf16) into this wave's LDS tile
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l) {
                if (KV == DT_BF16) {
                    *(uint4*)(stage + lds_off<HD>(vrow[l], vcb[l])) = vr[s][l];
                } else {
                    const bf16x8 v0 = kv_operand_from_bytes<KV>(vr[s][l], 0);
                    const bf16x8 v1 = kv_operand_from_bytes<KV>(vr[s][l], 1);
                    *(bf16x8*)(stage + lds_off<HD>(vrow[l], vcb[l])) = v0;
                    *(bf16x8*)(stage + lds_off<HD>(vrow[l], vcb[l] + 1)) = v1;
                }
            }
            // scores S^T = K . Q^T
            f32x4 st = {0, 0, 0, 0};
#pragma unroll
            for (int c = 0; c < T::NCH; ++c) {
                bf16x8 kop;
                if constexpr (KV == DT_BF16) kop = kv_operand_from_bytes<KV>(kr[s][c], 0);
                else kop = kv_operand_from_bytes<KV>(kr[s][c / 2], c % 2);
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qhi[c], st, 0, 0, 0);
                if (QT == DT_F32) st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qlo[c], st, 0, 0, 0);
            }
            // refill this slot with the block kDepth ahead
            if (refill) issue(s, i + kDepth);

            // online softmax over this block's 16 tokens (base-2 domain)
            const float mult = QUANT ? a.scale_log2 * __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ksc), i))
                                     : a.scale_log2;
            float sv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sv[e] = st[e] * mult;
                if (valid < 16 && 4 * grp + e >= valid) sv[e] = -__builtin_inff();
            }
            float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            mx = fmaxf(mx, fshfl_xor(mx, 16));
            mx = fmaxf(mx, fshfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            float pe[4], psum = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pe[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
                psum += pe[e];
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
#pragma unroll
            for (int t = 0; t < T::NT; ++t) acc[t] *= alpha;

            const float vs = QUANT ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vsc), i))
                                   : 1.0f;
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) split_bf16(pe[e] * vs, hi[e], lo[e]);
            const s16x4 phi = {(short)hi[0], (short)hi[1], (short)hi[2], (short)hi[3]};
            const s16x4 plo = {(short)lo[0], (short)lo[1], (short)lo[2], (short)lo[3]};

            // O^T += V^T . P^T
#pragma unroll
            for (int t = 0; t < T::NT; ++t) {
                const s16x4 vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)(stage + trd[t]));
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, phi, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, plo, acc[t], 0, 0, 0);
            }
        };

        int it = 0;
        if (cnt >= 2 * kDepth) {
            // prologue and steady state issue unconditionally and in slot
            // order (the scheduling barriers keep the prologue's independent
            // loads from being reordered), so at the loop head the newest loads
            // are always the other slots' and each block waits only for itself
#pragma unroll
            for (int s = 0; s < kDepth; ++s) {
                issue(s, s);
                __builtin_amdgcn_sched_barrier(0);
            }
            for (; it + 2 * kDepth <= cnt; it += kDepth) {
#pragma unroll
                for (int s = 0; s < kDepth; ++s) consume(s, it + s, true);
            }
        } else {
#pragma unroll
            for (int s = 0; s < kDepth; ++s)
                if (s < cnt) issue(s, s);
        }
        // drain: fewer than 2 * kDepth blocks remain, their first loads issued
#pragma unroll
        for (int k = 0; k < 2 * kDepth; ++k)
            if (it + k < cnt) consume(k % kDepth, it + k, it + k + kDepth < cnt);
    }

    // ---- merge the four waves' states through LDS
    float l_tot = l_run + fshfl_xor(l_run, 16);
    l_tot += fshfl_xor(l_tot, 32);
    if (bad) l_tot = __builtin_nanf("");
    __syncthreads();   // staging area is reused below
    float* lo_buf = (float*)smem;                        // [4][16][OROW]
    float* ml_buf = (float*)(smem + 4 * 16 * OROW * 4);  // [4][16][2]
    if (col < g) {
#pragma unroll
        for (int t = 0; t < T::NT; ++t)
            *(f32x4*)(lo_buf + (wave * 16 + col) * OROW + 16 * t + 4 * grp) = acc[t];
        if (grp == 0) {
            ml_buf[(wave * 16 + col) * 2 + 0] = m_run;
            ml_buf[(wave * 16 + col) * 2 + 1] = l_tot;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < g * HD; idx += kAttnThreads) {
        const int h = idx / HD, d = idx % HD;
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_buf[(w * 16 + h) * 2]);
        float L = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = ml_buf[(w * 16 + h) * 2];
            const float sc = mw == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            L += sc * ml_buf[(w * 16 + h) * 2 + 1];
            o += sc * lo_buf[(w * 16 + h) * OROW + d];
        }
        const int64_t row = (int64_t)b * a.n_q + j * g + h;
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

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
    dim3 grid(a.P, a.n_kv, a.B);
    dim3 block(kAttnThreads);
#define PDA_LAUNCH(HD, KV, QT) \
    hipLaunchKernelGGL((k_attn_mfma<HD, KV, QT>), grid, block, 0, s, a)
#define PDA_BY_Q(HD, KV)                          \
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
