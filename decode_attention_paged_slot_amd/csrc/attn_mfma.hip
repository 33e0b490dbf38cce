// attn_mfma.hip -- paged single-token decode attention on CDNA4 matrix cores,
// for 16-bit (bf16) and 8-bit (fp8 e4m3 / int8 + per-block scale) caches, and
// for 4-bit caches (codes with per-channel key scales and per-token value
// scales; each row's open block stays in a bf16 residual window, read by the
// merge; SoK paper section 2.3). With the step's new K/V rows (the fused
// decode step), the waves that stream a row's blocks also append them.
//
// What is computed (sections 9.4-9.5 of "9 Decode and KV Cache"; SoK paper
// section 1.1): for every sequence b, KV head j and the g = n_q / n_kv query
// heads h of its group, softmax(scale * q_h . K_t) over t < n_b, applied to
// V_t, where token t lives at (block_table[b][t / 16], t % 16). One read of
// each (block, head) K/V tile serves all g query heads (the GQA reuse that
// gives 2 g / w_kv FLOP per byte), scores never leave registers.
//
// Work decomposition. A segment is one (sequence b, KV head j) pair with
// nblk_b = ceil(n_b / 16) blocks; segments are laid end to end (b major, j
// minor) on one flattened axis of T = n_kv * sum_b nblk_b blocks.
//  - Split mode: the axis is cut into NW equal contiguous ranges (NW capped
//    at T), one per wave (four independent waves per workgroup, about one
//    workgroup per compute unit), so every wave streams the same number of
//    blocks however ragged the batch is. A wave's range covers pieces of one or more
//    segments; its load pipeline runs across segment boundaries. A piece
//    that is a whole segment is normalised and written to the output; any
//    other piece writes a partial (normalised output, base-2 max, sum) to
//    slot segment + wave, and the merge kernel combines the pieces of each
//    split segment, whose wave range [first, last] the wave that starts the
//    segment records. Each workgroup first computes the per-sequence block
//    prefix sums from context_lens in LDS (no host round trip).
//  - Unsplit mode: wave w streams segment w alone and writes its output.
//
// Per 16-token block and wave:
//   S^T[16 tok][16 heads] = K_tile[16][d_h] . Q^T[d_h][16]  -- MFMA 16x16x32 bf16;
//     a bf16 K tile is loaded with contiguous 1 KiB-per-instruction loads and
//     passed through an XOR-swizzled LDS tile into the A-operand layout; an
//     8-bit tile goes from HBM straight into the A operand (lane (t, grp)
//     holds contiguous bytes of token row t) and is converted in registers.
//     Q sits in the B operand with the same element order (the contraction
//     order over d_h is free).
//   The S^T accumulator layout puts 4 tokens of one head in each lane, which
//   is exactly the B-operand layout of the value product, so the
//   probabilities never move between lanes.
//   O^T[d_h][16 heads] += [V^T | V^T][d_h][32] . [P_hi; P_lo][32][16]  -- one
//     MFMA 16x16x32 bf16 per 16 columns; V is staged through LDS (XOR-swizzled
//     rows, conflict-free) and read back transposed with ds_read_b64_tr_b16.
//     P is split into bf16 hi + lo parts so the weights keep ~16 bits; the
//     doubled V operand folds both parts into one instruction. Q in fp32 is
//     split the same way.
//   8-bit caches are converted to bf16 in registers (exact), the K scale is
//   folded into the score multiplier and the V scale into P.
// Loads run `kDepth` blocks ahead of the math in each wave and are marked
// non-temporal (every cache byte is read once per step).
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

#ifndef PDA_ATTN_DEPTH
#define PDA_ATTN_DEPTH 2
#endif
#ifndef PDA_INT4_DEPTH
#define PDA_INT4_DEPTH 4
#endif
constexpr int kDepth = PDA_ATTN_DEPTH;   // blocks in flight per wave beyond the one being consumed
// 4-bit tiles are a quarter of a bf16 tile: more of them in flight per wave
// keep as many bytes outstanding
constexpr int kDepthInt4 = PDA_INT4_DEPTH;
constexpr float kSlack = 8.0f;   // lazy-rescaling threshold (weights < 2^8)

template <int HD, int KV>
struct Tr {
    static constexpr bool I4 = KV == DT_INT4;
    static constexpr int W = (KV == DT_BF16) ? 2 : 1;   // bytes per cached element (16/8-bit)
    static constexpr int ROWB = I4 ? HD / 2 : HD * W;   // bytes per token row
    static constexpr int TILEB = 16 * ROWB;             // bytes per (block, head) tile
    static constexpr int LOADS = I4 ? 1 : TILEB / 1024; // 16-B loads per lane per tile
    static constexpr int LB = TILEB / 64;               // 4-bit: tile bytes per lane (16 or 8)
    static constexpr int NCH = HD / 32;                 // QK k-chunks
    static constexpr int NT = HD / 16;                  // PV output tiles
    static constexpr int LROW = HD * 2;                 // bytes per bf16 LDS row
    static constexpr int LTILE = 16 * LROW;
    static constexpr int CPR = HD / 8;                  // 16-B chunks per LDS row
    static constexpr int RPS = 256 / LROW;              // LDS rows per 256 B
    static constexpr int CPRB = ROWB / 16;              // 16-B chunks per cache row
};

// First element of QK chunk c held by lane group grp (8 consecutive elements).
template <int HD, int KV>
__device__ __forceinline__ constexpr int dmap(int c, int grp) {
    return KV == DT_BF16   ? 32 * c + 8 * grp
           : KV == DT_INT4 ? (HD / 4) * grp + 8 * c   // lane group grp: channels of its 16-B load
                           : 64 * (c / 2) + 16 * grp + 8 * (c % 2);
}

__device__ __forceinline__ uint4 ld16(const char* p) { return *(const uint4*)p; }

// global-address-space views, for loads whose base comes out of an asm
// statement (a plain pointer there would be taken as a flat address)
typedef __attribute__((address_space(1))) const char gchar;
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const u32x2 gu32x2;
typedef __attribute__((address_space(1))) const f32x4 gf32x4;

// Streaming 16-B load of cache data: a private K/V byte is read exactly once
// per step, so the load is marked non-temporal and does not displace
// reusable lines from the caches (measured on MI355X: random 4 KiB tile reads
// 5.95 -> 6.66 TB/s). Blocks the caller marks as shared by many rows are read
// with ordinary loads instead, so their later readers hit in L2 / MALL.
__device__ __forceinline__ uint4 ld16_stream(const char* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}


// The new row's elements this lane holds (8 bytes of the source row: 4 bf16
// or 2 fp32 values) -> their cache codes, encoded with the destination
// block's reciprocal scale exactly as the quantized append encodes them:
// y = x * fp32(1 / scale), round to nearest even, saturate. Returns the codes
// packed low byte first (4 or 2 of them).
template <int KV>
__device__ __forceinline__ uint32_t encode_lane(uint2 w, int src_dtype, float inv) {
    float x[4];
    int n;
    if (src_dtype == DT_F32) {
        x[0] = __uint_as_float(w.x);
        x[1] = __uint_as_float(w.y);
        n = 2;
    } else {
        x[0] = bf16_lo_to_f32(w.x);
        x[1] = bf16_hi_to_f32(w.x);
        x[2] = bf16_lo_to_f32(w.y);
        x[3] = bf16_hi_to_f32(w.y);
        n = 4;
    }
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e < n) {
            const float y = __fmul_rn(x[e], inv);
            const uint32_t code = KV == DT_FP8 ? quant_fp8_e4m3(y) : ((uint32_t)quant_int8(y) & 0xFFu);
            packed |= code << (8 * e);
        }
    }
    return packed;
}

// Per-block metadata, lane i of a 64-block batch describing block i.
//   info bit 4 the row has a shared prefix (its pieces always go through
//   the merge), bit 5 first block of its segment, bit 6 last block of its
//   segment, bit 7 shared (cache-retaining loads), bits 8.. segment index.
// A segment lists only the blocks holding attended positions (all blocks of
// the row, or its sink and window blocks with a sliding window).
struct Meta {
    int id;      // physical block, or -1 when the table entry is unmapped
                 // (bf16: the raw table entry, checked where used)
    int tile;    // (block, head) tile index id * n_kv + j (block 0 when
                 // unmapped); bf16: the head j
    int info;
    int mask;    // attended positions of the block (bit k: token k)
    float ksc, vsc;
};

template <int HD, int KV, int QT>
__global__ void __launch_bounds__(kAttnThreads, KV == DT_BF16 ? 1 : 2) k_attn_mfma(AttnArgs a) {
    constexpr int kDepth = KV == DT_INT4 ? kDepthInt4 : pda::kDepth;   // this kernel's depth
    using T = Tr<HD, KV>;
    constexpr bool QUANT = KV == DT_FP8 || KV == DT_INT8;   // 8-bit, per-(block, head) scales
    // bf16: block metadata keeps the raw table entry and the head rather
    // than the checked id and tile index (8-bit caches need the tile there
    // for their scale loads; loading the scales with each block's tiles
    // instead made the 8-bit calls 30% slower)
    constexpr bool kLazyId = KV == DT_BF16;
    constexpr bool I4 = KV == DT_INT4;   // 4-bit: per-channel K and per-token V scales
    // per wave: the V tile (bf16) and, for bf16 caches, the K tile
    constexpr bool KST = KV == DT_BF16;
    // (the 4-bit kernel stages the V tiles of two blocks per step)
    __shared__ __attribute__((aligned(16))) char stage_all[4 * T::LTILE * ((KST || I4) ? 2 : 1)];
    // fused decode step: per wave, the new K and V rows (up to 512 B each)
    __shared__ __attribute__((aligned(16))) char newrow_all[4 * 2 * 512];
    __shared__ int wsum[4], wsumu[4];
    extern __shared__ int dyn_lds[];
    int* pre = dyn_lds;             // [B + 1] exclusive prefix of blocks per sequence
    int* nn = dyn_lds + a.B + 1;    // [B] context length, -1 for an invalid one
    int* preu = dyn_lds + 2 * a.B + 1;   // [B + 1] exclusive prefix of split units per sequence
    int* plen = dyn_lds + 3 * a.B + 2;   // [B] shared-prefix lengths as given (prefix calls only)

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int col = lane & 15;   // token row (A operand) / query head (B, D)
    const int grp = lane >> 4;
    const int g = a.g;
    const int B = a.B;
    const int n_kv = a.n_kv;

    // ---- per-sequence block counts and their exclusive prefixes (LDS): in
    // blocks, and in split units, where every non-empty segment also counts
    // seg_cost units for its fixed costs (query load, partial write), so that
    // waves crossing many short segments get fewer blocks
    // (4-bit: no segment cost, so that units are blocks and cuts fall between pairs)
    const int C = I4 ? 0 : a.seg_cost;
    {
        const int R = (B + kAttnThreads - 1) / kAttnThreads;
        const int r0 = threadIdx.x * R;
        auto seg_blocks = [&](int b, int n) {
            // with a shared prefix, only the row's blocks after it are streamed here
            const int pl = a.prefix_lens == nullptr
                               ? (n < 0 || n > a.max_blocks * 16 ? -1 : 0)
                               : row_prefix_len(n, a.prefix_lens[b], a.max_blocks,
                                                a.prefix_blocks);
            // 4-bit: the encoded blocks (the open one is a piece of its own),
            // padded to an even count with one fully masked block, so that
            // every segment starts at an even position of the block axis
            if (I4) return pl < 0 ? -1 : ((n / 16) + 1) & ~1;
            return pl < 0 ? -1 : row_blocks(n, a.window, a.sinks).count - pl;
        };
        int local = 0, localu = 0;
        for (int r = 0; r < R; ++r) {
            const int b = r0 + r;
            if (b < B) {
                const int n = a.context_lens[b];
                const int c = seg_blocks(b, n);
                if (a.prefix_lens != nullptr) plen[b] = a.prefix_lens[b];
                nn[b] = c < 0 ? -1 : n;
                const int cb = max(c, 0);
                local += cb;
                localu += cb + (cb > 0 ? C : 0);
            }
        }
        int incl = local, inclu = localu;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            const int yu = __shfl_up(inclu, o, 64);
            if (lane >= o) {
                incl += y;
                inclu += yu;
            }
        }
        if (lane == 63) {
            wsum[wave] = incl;
            wsumu[wave] = inclu;
        }
        __syncthreads();
        int run = incl - local, runu = inclu - localu;
        for (int w = 0; w < wave; ++w) {
            run += wsum[w];
            runu += wsumu[w];
        }
        for (int r = 0; r < R; ++r) {
            const int b = r0 + r;
            if (b < B) {
                pre[b] = run;
                preu[b] = runu;
                const int cb = nn[b] < 0 ? 0 : max(seg_blocks(b, nn[b]), 0);
                run += cb;
                runu += cb + (cb > 0 ? C : 0);
            }
        }
        if (threadIdx.x == kAttnThreads - 1) {
            pre[B] = run;
            preu[B] = runu;
        }
        __syncthreads();
    }
    const int64_t T_all = (int64_t)n_kv * pre[B];
    const int64_t T_u = (int64_t)n_kv * preu[B];
    // never more ranges than units: every range in use is non-empty, so the
    // pieces of a segment come from consecutive waves without gaps
    // (4-bit: ranges are cut between pairs of blocks, T_u / 2 pairs)
    const int NW = (int)max((int64_t)1, min((int64_t)a.nw, I4 ? T_u / 2 : T_u));
    const int wg = blockIdx.x * 4 + wave;   // global wave index

    // first block position at or after unit u: segment s of row b spans units
    // [U, U + C + nb), its fixed-cost units first, then one unit per block
    auto unit_to_block = [&](int64_t u) -> int64_t {
        if (u >= T_u) return T_all;
        int l = 0, r = B - 1;   // last sequence whose first unit is <= u (non-empty)
        while (l < r) {
            const int mid = (l + r + 1) >> 1;
            if ((int64_t)n_kv * preu[mid] <= u) l = mid;
            else r = mid - 1;
        }
        const int nb = pre[l + 1] - pre[l];
        const int64_t r0 = u - (int64_t)n_kv * preu[l];
        const int j = (int)(r0 / (nb + C));
        const int off = (int)(r0 - (int64_t)j * (nb + C));
        return (int64_t)n_kv * pre[l] + (int64_t)j * nb + max(0, off - C);
    };

    // ---- this wave's range [lo, hi) of the flattened block axis
    int64_t lo = 0, hi = 0, lo_u = 0, hi_u = 0;
    if (a.split) {
        if (wg < NW) {
            if (I4) {
                lo_u = 2 * ((int64_t)wg * (T_u / 2) / NW);
                hi_u = 2 * ((int64_t)(wg + 1) * (T_u / 2) / NW);
            } else {
                lo_u = (int64_t)wg * T_u / NW;
                hi_u = (int64_t)(wg + 1) * T_u / NW;
            }
            lo = C == 0 ? lo_u : unit_to_block(lo_u);   // with no segment cost, units are blocks
            hi = C == 0 ? hi_u : unit_to_block(hi_u);
        }
    } else if (wg < B * n_kv) {
        const int b = wg / n_kv, j = wg - (wg / n_kv) * n_kv;
        const int nb = pre[b + 1] - pre[b];
        lo = (int64_t)n_kv * pre[b] + (int64_t)j * nb;
        hi = lo + nb;
    }

    auto write_rows = [&](int64_t row0, int nrows, float v) {
        for (int idx = lane; idx < nrows * HD; idx += 64) {
            const int64_t o = row0 * HD + idx;
            if (a.out_dtype == DT_F32) ((float*)a.out)[o] = v;
            else ((uint16_t*)a.out)[o] = (uint16_t)f32_to_bf16_rne(v);
        }
    };

    // ---- fused 4-bit decode step: the append's work (the 4-bit cache's
    // append path with its residual window, SoK paper section 2.3), done by
    // the waves that own it before they stream. The new token of (row b,
    // KV head j) goes to residual slot (n - 1) % 16 (a bit copy); when it
    // fills the block, the block's 16 tokens (15 residual rows and the new
    // one) are encoded into the cache: keys with the per-channel scales,
    // values with one scale per token (amax / 7 over the token's channels,
    // 1 if that is 0 or not finite), codes RNE(x * fp32(1 / s)) clamped to
    // [-7, 7]. The arithmetic is the separate append's, so both give the
    // same bits.
    auto resid_write = [&](int b, int j) {
        const int r = (nn[b] - 1) & 15;
        const int64_t sj = (int64_t)b * n_kv + j;
        const uint32_t* kn = (const uint32_t*)a.k_new + sj * (HD / 2);
        const uint32_t* vn = (const uint32_t*)a.v_new + sj * (HD / 2);
        uint32_t* kd = (uint32_t*)a.k_res + (sj * 16 + r) * (HD / 2);
        uint32_t* vd = (uint32_t*)a.v_res + (sj * 16 + r) * (HD / 2);
        for (int x = lane; x < HD / 2; x += 64) {
            kd[x] = kn[x];
            vd[x] = vn[x];
        }
    };
    // encode the block completed by the new token of (b, j) into physical
    // block pb: lane (token t = col, quarter grp) encodes channels
    // grp * d_h / 4 .. +d_h / 4 of token t, the bytes it streams later
    auto encode_fill = [&](int b, int j, int pb) {
        constexpr int CPL = HD / 4;   // channels per lane
        float* kinv = (float*)(stage_all + wave * T::LTILE);   // fp32(1 / k_scale), this wave's stage
        for (int c = lane; c < HD; c += 64) kinv[c] = __fdiv_rn(1.0f, a.k_scale[(int64_t)j * HD + c]);
        const int64_t sj = (int64_t)b * n_kv + j;
        const uint16_t* ks = (col == 15 ? (const uint16_t*)a.k_new + sj * HD
                                        : (const uint16_t*)a.k_res + (sj * 16 + col) * HD) + grp * CPL;
        const uint16_t* vs = (col == 15 ? (const uint16_t*)a.v_new + sj * HD
                                        : (const uint16_t*)a.v_res + (sj * 16 + col) * HD) + grp * CPL;
        float kx[CPL], vx[CPL];
#pragma unroll
        for (int q = 0; q < CPL / 8; ++q) {
            const uint4 kw = *(const uint4*)(ks + 8 * q);
            const uint4 vw = *(const uint4*)(vs + 8 * q);
            const uint32_t ka[4] = {kw.x, kw.y, kw.z, kw.w}, va[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kx[8 * q + 2 * e] = bf16_lo_to_f32(ka[e]);
                kx[8 * q + 2 * e + 1] = bf16_hi_to_f32(ka[e]);
                vx[8 * q + 2 * e] = bf16_lo_to_f32(va[e]);
                vx[8 * q + 2 * e + 1] = bf16_hi_to_f32(va[e]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): kinv is in LDS
        __builtin_amdgcn_wave_barrier();
        uint32_t kp[CPL / 8], vp[CPL / 8];
#pragma unroll
        for (int q = 0; q < CPL / 8; ++q) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = grp * CPL + 8 * q + i;
                const uint32_t lo = quant_int4_nibble(__fmul_rn(kx[8 * q + i], kinv[c]));
                const uint32_t hi = quant_int4_nibble(__fmul_rn(kx[8 * q + 4 + i], kinv[c + 4]));
                w |= (lo | (hi << 4)) << (8 * i);
            }
            kp[q] = w;
        }
        float amax = 0.0f, nf = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float v = fabsf(vx[c]);
            if (!(v <= 3.402823466e38f)) nf = 1.0f;   // NaN or infinite
            amax = fmaxf(amax, v);
        }
        amax = max_rows4(amax);   // the token's four lanes
        nf = max_rows4(nf);
        const float sc = (nf == 0.0f && amax > 0.0f) ? __fdiv_rn(amax, 7.0f) : 1.0f;
        const float inv = __fdiv_rn(1.0f, sc);
#pragma unroll
        for (int q = 0; q < CPL / 8; ++q) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = quant_int4_nibble(__fmul_rn(vx[8 * q + i], inv));
                const uint32_t hi = quant_int4_nibble(__fmul_rn(vx[8 * q + 4 + i], inv));
                w |= (lo | (hi << 4)) << (8 * i);
            }
            vp[q] = w;
        }
        const int64_t tbyte = ((int64_t)pb * n_kv + j) * T::TILEB + col * T::ROWB + grp * T::LB;
        if constexpr (CPL / 8 == 4) {
            *(uint4*)((char*)a.k + tbyte) = make_uint4(kp[0], kp[1], kp[2], kp[3]);
            *(uint4*)((char*)a.v + tbyte) = make_uint4(vp[0], vp[1], vp[2], vp[3]);
        } else {
            *(uint2*)((char*)a.k + tbyte) = make_uint2(kp[0], kp[1]);
            *(uint2*)((char*)a.v + tbyte) = make_uint2(vp[0], vp[1]);
        }
        if (grp == 0) ((float*)a.v_scale)[((int64_t)pb * n_kv + j) * 16 + col] = sc;
    };

    // ---- sequences without blocks (empty, or invalid length): zero / NaN rows.
    // Split mode: such a sequence sits at unit n_kv * preu[b]; the wave whose
    // unit range holds it owns it (the last wave also owns the unit T_u).
    // Unsplit mode: the wave of each of its segments.
    if (a.split) {
        if (wg < NW) {
            const int64_t hi_ext = (wg == NW - 1) ? T_u + 1 : hi_u;
            int l = 0, r = B;
            while (l < r) {
                const int mid = (l + r) >> 1;
                if ((int64_t)n_kv * preu[mid] >= lo_u) r = mid;
                else l = mid + 1;
            }
            for (int b = l; b < B && (int64_t)n_kv * preu[b] < hi_ext; ++b) {
                if (pre[b + 1] != pre[b]) continue;
                write_rows((int64_t)b * a.n_q, a.n_q, nn[b] < 0 ? __builtin_nanf("") : 0.0f);
                for (int jj = lane; jj < n_kv; jj += 64)
                    a.seg_info[(int64_t)b * n_kv + jj] = make_int2(0, -1);
                // fused 4-bit step: a row shorter than a block still appends
                if (I4 && a.k_new != nullptr && nn[b] > 0)
                    for (int jj = 0; jj < n_kv; ++jj) resid_write(b, jj);
            }
        }
    } else if (wg < B * n_kv && hi == lo) {
        write_rows((int64_t)wg * g, g, nn[wg / n_kv] < 0 ? __builtin_nanf("") : 0.0f);
    }

    const int cnt = (int)(hi - lo);
    if (cnt <= 0) return;

    // fused 4-bit step, the segments this wave streams: the wave holding a
    // segment's first block writes its new token to the residual window, and
    // the wave holding a block the new token completes encodes it before
    // streaming (its stores are complete before its own loads of the tile)
    if (I4 && a.k_new != nullptr) {
        bool wrote = false;
        for (int64_t pos = lo; pos < hi;) {
            int l = 0, r = B - 1;   // the sequence holding position pos
            while (l < r) {
                const int mid = (l + r + 1) >> 1;
                if ((int64_t)n_kv * pre[mid] <= pos) l = mid;
                else r = mid - 1;
            }
            const int b = l, nb = pre[b + 1] - pre[b];
            const int j = (int)((pos - (int64_t)n_kv * pre[b]) / nb);
            const int64_t S = (int64_t)n_kv * pre[b] + (int64_t)j * nb;   // segment start
            if (S >= lo) resid_write(b, j);
            const int n = nn[b];
            if (n >= 16 && (n & 15) == 0) {
                const int64_t F = S + (n >> 4) - 1;   // the block the new token completes
                if (F >= lo && F < hi) {
                    const int pb = a.block_table[(int64_t)b * a.max_blocks + (n >> 4) - 1];
                    if (pb >= 0 && pb < a.num_blocks) {
                        encode_fill(b, j, pb);
                        wrote = true;
                    }
                }
            }
            pos = S + nb;
        }
        if (wrote) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // ---- per-block metadata of batch `batch` (64 blocks from lo + 64 * batch)
    auto load_meta = [&](int batch) {
        Meta m{-1, 0, 0, 0, 1.0f, 1.0f};
        const int64_t f = lo + (int64_t)batch * 64 + lane;
        if (f < hi) {
            const int x = (int)f;
            int l = 0, r = B - 1;   // last sequence whose first position is <= x
            while (l < r) {
                const int mid = (l + r + 1) >> 1;
                if (n_kv * pre[mid] <= x) l = mid;
                else r = mid - 1;
            }
            const int b = l;
            const int nb = pre[b + 1] - pre[b];
            const int r0 = x - n_kv * pre[b];
            const int j = r0 / nb;
            const int bl = r0 - j * nb;   // attended-block index within the row
            // rows with a shared prefix: their first pl blocks belong to the
            // prefix pass, this pass starts after them (no window there)
            // (from LDS: a global load here would be waited for, with every
            // load issued before it, before the block lookup goes out)
            const int pl = a.prefix_lens == nullptr ? 0 : plen[b];
            const int blk = row_block_logical(row_blocks(nn[b], a.window, a.sinks), bl) + pl;
            // 4-bit: the pad block that evens a segment's block count is
            // fully masked and reads block 0 (no table lookup, no poison)
            const bool pad = I4 && bl >= (nn[b] >> 4);
            int id = pad ? 0 : a.block_table[(int64_t)b * a.max_blocks + blk];
            const int seg = b * n_kv + j;
            if constexpr (kLazyId) {
                // the id is range-checked where it is used (issue, consume),
                // so nothing here waits for the table load and a second
                // batch's lookups are in flight with the first's
                m.id = id;
                m.tile = j;
            } else {
                if (id < 0 || id >= a.num_blocks) id = -1;
                m.id = id;
                m.tile = (id < 0 ? 0 : id) * n_kv + j;
            }
            // bit 4: the row's pieces always go to the merge (a shared
            // prefix, or a 4-bit cache's non-empty residual window)
            const bool merged = pl > 0 || (a.extra_pieces > 0 && (nn[b] & 15) != 0);
            m.info = (merged << 4) | ((bl == 0) << 5) | ((bl == nb - 1) << 6) |
                     ((blk < a.reuse_blocks) << 7) | (seg << 8);
            m.mask = pad ? 0 : (int)block_token_mask(blk, nn[b], a.window, a.sinks);
            if (QUANT && id >= 0) {
                // ordinary loads: the n_kv heads of a block share these
                // lines, so they are worth keeping in L2 (streaming them
                // measured slower, unlike the 4-bit value scales below)
                m.ksc = a.k_scale[m.tile];
                m.vsc = a.v_scale[m.tile];
            }
        }
        return m;
    };

    // ---- query operands (B operand of S^T = K . Q^T): lane (h, grp), for
    // the g query rows of segment `seg` (rows seg * g .. seg * g + g - 1)
    bf16x8 qhi[T::NCH], qlo[T::NCH];
    // 4-bit: the per-channel key scales and the base-2 softmax scale are
    // folded into the queries, q' = q * (k_scale[j][:] * scale_log2) in fp32,
    // split into bf16 hi + lo; the K operand holds 136 + code, so every score
    // carries the offset cq = 136 * sum_d q'_d (computed from the very hi and
    // lo values multiplied). The score products start from -(cq + m_use4)
    // (sinit), so they come out in the log2 domain relative to the piece's
    // reference maximum, with no vector instruction per score.
    float cq = 0.0f;
    float m_use4 = 0.0f;                  // the reference the 4-bit scores are relative to
    float sinit = 0.0f;                   // -(cq + m_use4)
    float thr4 = -__builtin_inff();       // rescale threshold: kSlack, or -inf before the first max
    // 4-bit: a segment's query words and key scales are fetched (q_fetch)
    // and then combined (load_q with fetched = true) in two steps, so that
    // the first segment's fetch is in flight together with the first tiles
    // while its arithmetic waits only for itself
    float4 qw[T::NCH][2], kw4[T::NCH][2];
    auto q_fetch = [&](int seg) {
        if constexpr (I4) {
            const bool live = col < g;
            const int64_t qrow = ((int64_t)seg * g + (live ? col : 0)) * HD;
#pragma unroll
            for (int c = 0; c < T::NCH; ++c) {
                const int d0 = dmap<HD, KV>(c, grp);
                if (QT == DT_BF16) {
                    const uint4 w = live ? ld16((const char*)a.q + (qrow + d0) * 2)
                                         : make_uint4(0, 0, 0, 0);
                    qw[c][0] = __builtin_bit_cast(float4, w);
                } else {
                    qw[c][0] = live ? *(const float4*)((const float*)a.q + qrow + d0)
                                    : make_float4(0, 0, 0, 0);
                    qw[c][1] = live ? *(const float4*)((const float*)a.q + qrow + d0 + 4)
                                    : make_float4(0, 0, 0, 0);
                }
                const float* ks = a.k_scale + (int64_t)(seg % n_kv) * HD + d0;
                kw4[c][0] = *(const float4*)ks;
                kw4[c][1] = *(const float4*)(ks + 4);
            }
        }
    };
    auto load_q = [&](int seg, bool fetched = false) {
        if (I4 && !fetched) q_fetch(seg);
        const bool live = col < g;
        const int64_t qrow = ((int64_t)seg * g + (live ? col : 0)) * HD;
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < T::NCH; ++c) {
            const int d0 = dmap<HD, KV>(c, grp);
            if constexpr (I4) {
                float f[8];
                if (QT == DT_BF16) {
                    const uint4 w = __builtin_bit_cast(uint4, qw[c][0]);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        f[2 * k] = bf16_lo_to_f32(ws[k]);
                        f[2 * k + 1] = bf16_hi_to_f32(ws[k]);
                    }
                } else {
                    f[0] = qw[c][0].x; f[1] = qw[c][0].y; f[2] = qw[c][0].z; f[3] = qw[c][0].w;
                    f[4] = qw[c][1].x; f[5] = qw[c][1].y; f[6] = qw[c][1].z; f[7] = qw[c][1].w;
                }
                const float4 k0 = kw4[c][0], k1 = kw4[c][1];
                const float sl = a.scale_log2;
                f[0] *= k0.x * sl; f[1] *= k0.y * sl; f[2] *= k0.z * sl; f[3] *= k0.w * sl;
                f[4] *= k1.x * sl; f[5] *= k1.y * sl; f[6] *= k1.z * sl; f[7] *= k1.w * sl;
                uint32_t h16[8], l16[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    split_bf16(f[e], h16[e], l16[e]);
                    part += __uint_as_float(h16[e] << 16) + __uint_as_float(l16[e] << 16);
                }
                u32x4 hv = {h16[0] | (h16[1] << 16), h16[2] | (h16[3] << 16),
                            h16[4] | (h16[5] << 16), h16[6] | (h16[7] << 16)};
                u32x4 lv = {l16[0] | (l16[1] << 16), l16[2] | (l16[3] << 16),
                            l16[4] | (l16[5] << 16), l16[6] | (l16[7] << 16)};
                qhi[c] = __builtin_bit_cast(bf16x8, hv);
                qlo[c] = __builtin_bit_cast(bf16x8, lv);
            } else if (QT == DT_BF16) {
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
        if constexpr (I4) {
            cq = kInt4Bias * sum_rows4(part);
            sinit = -(cq + m_use4);
        }
    };

    // ---- per-piece online-softmax state
    float m_run = -__builtin_inff();
    float l_run = 0.0f;
    f32x4 acc[T::NT];
#pragma unroll
    for (int t = 0; t < T::NT; ++t) acc[t] = f32x4{0, 0, 0, 0};
    // 4-bit: sum of the value weights (hi + lo) fed to the value product, per
    // head, formed by one more matrix product of the weights with ones (every
    // row of it holds the column sums), so it costs no vector instructions
    f32x4 wfed = {0.0f, 0.0f, 0.0f, 0.0f};
    bool piece_bad = false;
    bool piece_whole = false;   // the current piece began at its segment's first block
    int q_seg = -1;

    char* stage = stage_all + wave * T::LTILE;
    char* kstage = stage_all + (4 + wave) * T::LTILE;   // used when KST
    constexpr int kStage2 = 4 * T::LTILE;               // 4-bit: the second V tile, after the first
    const char* kbase = (const char*)a.k;
    const char* vbase = (const char*)a.v;
    const int64_t head_stride = T::TILEB;
    const int64_t block_stride = (int64_t)n_kv * T::TILEB;

    // V row / chunk handled by this lane for load l of a tile
    int vrow[T::LOADS], vcb[T::LOADS];
#pragma unroll
    for (int l = 0; l < T::LOADS; ++l) {
        const int byte = 1024 * l + 16 * lane;
        vrow[l] = byte / T::ROWB;
        vcb[l] = ((byte % T::ROWB) / T::W) / 8;   // bf16 chunk of the first element
    }
    // Transposed-read addresses for the value operand of the packed product
    // O^T += [V^T | V^T] . [P_hi ; P_lo] (MFMA 16x16x32, K = 32 = the block's
    // 16 tokens twice): lane l must hold V^T[d = 16 t + l % 16][tokens
    // base + 0..7] with base = 0 for lane rows 0 and 2, 8 for rows 1 and 3.
    // ds_read_b64_tr_b16 hands each 16-lane row G the 4 panel rows its own
    // lanes address (lane L: token of panel row L / 4, columns
    // 16 t + 4 (L % 4) .. +3), so two reads (tokens base + 0..3, base + 4..7)
    // give the 8 tokens.
    // The addresses include this wave's tile base and are formed once here;
    // the empty asm makes each one opaque, so the compiler keeps it whole in
    // a register rather than re-adding base and offset every block.
    using lds_s16x4 = __attribute__((address_space(3))) s16x4;
    uint32_t trd0[T::NT], trd1[T::NT];
    const uint32_t stage_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)stage;
#pragma unroll
    for (int t = 0; t < T::NT; ++t) {
        const int base = (grp & 1) * 8, q4 = lane & 3;
        const int r0 = base + ((lane & 15) >> 2);
        trd0[t] = stage_lds + lds_off<HD>(r0, 2 * t + (q4 >> 1)) + 8 * (q4 & 1);
        trd1[t] = stage_lds + lds_off<HD>(r0 + 4, 2 * t + (q4 >> 1)) + 8 * (q4 & 1);
        asm volatile("" : "+v"(trd0[t]), "+v"(trd1[t]));
    }

    // metadata of the consumer's batch (A) and of the next one (Bm)
    Meta A = load_meta(0);
    Meta Bm = cnt > 64 ? load_meta(1) : Meta{-1, 0, 0, 0, 1.0f, 1.0f};
    int batchA = 0;
    auto meta_info = [&](int i) {
        const int v = (i >> 6) == batchA ? A.info : Bm.info;
        return __builtin_amdgcn_readlane(v, i & 63);
    };
    auto meta_tile = [&](int i) {
        const int v = (i >> 6) == batchA ? A.tile : Bm.tile;
        const int t = __builtin_amdgcn_readlane(v, i & 63);
        if constexpr (kLazyId) {
            const int vi = (i >> 6) == batchA ? A.id : Bm.id;
            const int id = __builtin_amdgcn_readlane(vi, i & 63);
            return ((unsigned)id < (unsigned)a.num_blocks ? id : 0) * n_kv + t;
        }
        return t;
    };

    // the consumed block always lies in batch A (the consumer moves to the
    // next batch first), so its fields need no batch select
    auto cur_id = [&](int i) {
        const int id = __builtin_amdgcn_readlane(A.id, i & 63);
        return (!kLazyId || (unsigned)id < (unsigned)a.num_blocks) ? id : -1;
    };
    auto cur_info = [&](int i) { return __builtin_amdgcn_readlane(A.info, i & 63); };
    auto cur_f = [&](float f, int i) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), i & 63));
    };
    auto cur_mask = [&](int i) { return (uint32_t)__builtin_amdgcn_readlane(A.mask, i & 63); };

    uint4 kr[kDepth][T::LOADS], vr[kDepth][T::LOADS];
    f32x4 vsr[kDepth];   // 4-bit: value scales of this lane's 4 tokens
    uint2 nkr[kDepth], nvr[kDepth];   // fused step: 8 B of the new K / V row per lane
    char* newk = newrow_all + wave * 1024;
    char* newv = newk + 512;
    const int new_rowb = HD * (a.new_dtype == DT_F32 ? 4 : 2);   // bytes per new row

    // Loads are never predicated (a partially filled final block is still a
    // whole allocated tile; its tail rows are masked after loading; an
    // unmapped entry loads block 0 and poisons its piece), so every refill
    // issues the same instructions and the waits before each block's math
    // only drain that block's loads.
    // 4-bit loads: this lane's byte offset in a tile and in its value scales
    uint32_t i4_off = col * T::ROWB + grp * T::LB, i4_soff = 16u * (uint32_t)grp;
    auto issue = [&](int s, int i) {
        // the (block, head) tile: its index comes with the block's metadata,
        // so no division by n_kv happens per block
        const int64_t tile = (uint32_t)meta_tile(i);
        const int info = meta_info(i);
        const char* kt = kbase + tile * head_stride;
        const char* vt = vbase + tile * head_stride;
        // bf16 K: contiguous 1 KiB per load instruction (staged through LDS
        // into the operand layout); 8-bit K: straight into the operand
        // registers, lane (t, grp) taking 16 B of token row t
        if constexpr (I4) {
            // 4-bit tile: lane (t, grp) takes the LB bytes of token row t
            // holding channels (d_h / 4) grp .. +d_h / 4, for K (straight
            // into the operand) and V (through LDS) alike, and the value
            // scales of its tokens 4 grp .. 4 grp + 3
            // The tile bases are wave-uniform; the empty asm pins them in
            // scalar registers, so each load takes base + the lane's 32-bit
            // offset and no 64-bit vector address is formed per load.
            // The lane offsets are redefined in place by the same asm, so
            // their zero extension is formed beside the loads rather than
            // hoisted, which is what lets the loads take that form.
            uint64_t kb = (uint64_t)kt, vb = (uint64_t)vt, sb = (uint64_t)(a.v_scale + tile * 16);
            asm volatile("" : "+s"(kb), "+s"(vb), "+s"(sb), "+v"(i4_off), "+v"(i4_soff));
            const uint32_t off = i4_off, soff = i4_soff;
            const gchar* kg = (const gchar*)kb;
            const gchar* vg = (const gchar*)vb;
            const gchar* sg = (const gchar*)sb;
            if constexpr (T::LB == 16) {
                const u32x4 kk = __builtin_nontemporal_load((const gu32x4*)(kg + off));
                const u32x4 vv = __builtin_nontemporal_load((const gu32x4*)(vg + off));
                kr[s][0] = make_uint4(kk.x, kk.y, kk.z, kk.w);
                vr[s][0] = make_uint4(vv.x, vv.y, vv.z, vv.w);
            } else {
                const u32x2 kk = __builtin_nontemporal_load((const gu32x2*)(kg + off));
                const u32x2 vv = __builtin_nontemporal_load((const gu32x2*)(vg + off));
                kr[s][0] = make_uint4(kk.x, kk.y, 0, 0);
                vr[s][0] = make_uint4(vv.x, vv.y, 0, 0);
            }
            // the value scales are streamed like the codes (only this wave
            // reads a tile's): as an ordinary load, this one made the
            // 70B-shape 4-bit step 10 us slower when it ran right after a
            // 1 GiB write, i.e. with the caches full of dirty lines (MI355X:
            // 82.7 against 72.7 us)
            vsr[s] = __builtin_nontemporal_load((const gf32x4*)(sg + soff));
            return;
        }
        const int koff = KST ? 16 * lane : col * T::ROWB + 16 * grp;
        const int kstep = KST ? 1024 : 64;
        if (a.k_new != nullptr && ((info >> 6) & 1)) {
            // the row's newest block (fused step): its new K / V rows are
            // fetched with the tile, one coalesced 8-B piece per lane, so the
            // patch does not wait on memory (a wave may patch many rows in a
            // row when segments are a single block)
            const int64_t nrow = (int64_t)((unsigned)info >> 8) * new_rowb;
            if (8 * lane < new_rowb) {
                nkr[s] = *(const uint2*)((const char*)a.k_new + nrow + 8 * lane);
                nvr[s] = *(const uint2*)((const char*)a.v_new + nrow + 8 * lane);
            }
        }
        if ((info >> 7) & 1) {
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l) kr[s][l] = ld16(kt + koff + kstep * l);
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l) vr[s][l] = ld16(vt + 1024 * l + 16 * lane);
        } else {
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l) kr[s][l] = ld16_stream(kt + koff + kstep * l);
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l) vr[s][l] = ld16_stream(vt + 1024 * l + 16 * lane);
        }
    };

    auto flush = [&](int seg, bool whole) {
        float l_tot = sum_rows4(l_run);
        // 4-bit: the V operand holds 136 + code, so the product carries
        // 136 * (sum of the weights it was fed); remove it
        const float off = I4 ? kInt4Bias * wfed[0] : 0.0f;
        if (piece_bad) l_tot = __builtin_nanf("");
        if (col < g) {
            const int64_t prow = whole ? (int64_t)seg * g + col : ((int64_t)seg + wg) * g + col;
            f32x4 r[T::NT];
            const float inv = l_tot != 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
            for (int t = 0; t < T::NT; ++t) r[t] = (I4 ? acc[t] - off : acc[t]) * inv;
            if (!whole) {
#pragma unroll
                for (int t = 0; t < T::NT; ++t)
                    *(f32x4*)(a.part_o + prow * HD + 16 * t + 4 * grp) = r[t];
                if (grp == 0) *(float2*)(a.part_ml + prow * 2) = make_float2(m_run, l_tot);
            } else if (a.out_dtype == DT_F32) {
#pragma unroll
                for (int t = 0; t < T::NT; ++t)
                    *(f32x4*)((float*)a.out + prow * HD + 16 * t + 4 * grp) = r[t];
            } else {
#pragma unroll
                for (int t = 0; t < T::NT; ++t) {
                    uint2 h;
                    h.x = f32_to_bf16_rne(r[t][0]) | (f32_to_bf16_rne(r[t][1]) << 16);
                    h.y = f32_to_bf16_rne(r[t][2]) | (f32_to_bf16_rne(r[t][3]) << 16);
                    *(uint2*)((uint16_t*)a.out + prow * HD + 16 * t + 4 * grp) = h;
                }
            }
        }
        m_run = -__builtin_inff();
        l_run = 0.0f;
        wfed = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (I4) {
            m_use4 = 0.0f;
            sinit = -cq;
            thr4 = -__builtin_inff();
        }
#pragma unroll
        for (int t = 0; t < T::NT; ++t) acc[t] = f32x4{0, 0, 0, 0};
        piece_bad = false;
    };

    // a new piece starts at a segment's first block or at the range's first
    auto piece_start = [&](int seg, bool seg_first) {
        piece_whole = seg_first;
        if (seg != q_seg) {
            load_q(seg);
            q_seg = seg;
        }
        if (a.split && seg_first && lane == 0) {
            // record the waves covering this segment for the merge: the last
            // is the wave holding the segment's last unit
            const int b = seg / n_kv, j = seg - (seg / n_kv) * n_kv;
            const int64_t end_u =
                (int64_t)n_kv * preu[b] + (int64_t)(j + 1) * (pre[b + 1] - pre[b] + C);
            const int last_wave = I4 ? (int)((((end_u - 1) / 2 + 1) * NW - 1) / (T_u / 2))
                                     : (int)((end_u * NW - 1) / T_u);
            a.seg_info[seg] = make_int2(wg, last_wave);
        }
    };

    // the consumer moves to the next metadata batch when block i lies in it
    auto enter = [&](int i) {
        if ((i >> 6) != batchA) {
            A = Bm;
            ++batchA;
            if ((batchA + 1) * 64 < cnt) Bm = load_meta(batchA + 1);
        }
    };

    // P split into bf16 hi + lo (the weights keep ~16 bits). Lane (h, G)
    // holds tokens 4 G .. 4 G + 3 of head h as H_G (hi) and L_G (lo); the
    // packed B operand needs, per lane row G, k = 8 G .. 8 G + 7 = [H0 H1],
    // [H2 H3], [L0 L1], [L2 L3]: a permlane32 swap of (H, L) then a
    // permlane16 swap regroups them.
    auto pack_p = [&](const float (&w)[4]) -> bf16x8 {
        uint32_t H[2], L[2];
        split_bf16x2(w[0], w[1], H[0], L[0]);
        split_bf16x2(w[2], w[3], H[1], L[1]);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const auto x = __builtin_amdgcn_permlane32_swap(H[q], L[q], false, false);
            const auto y = __builtin_amdgcn_permlane16_swap(x[0], x[1], false, false);
            H[q] = y[0];
            L[q] = y[1];
        }
        const u32x4 pb4 = {H[0], H[1], L[0], L[1]};
        return __builtin_bit_cast(bf16x8, pb4);
    };

    // 4-bit: the scores come out relative to m_use4. When some head's
    // maximum exceeds its reference by more than kSlack (the test against
    // thr4), the reference moves as in the other caches, and this step's
    // scores are shifted to the new one.
    auto rescale4 = [&](float lmx, auto& sv) {
        const float mx = max_rows4(lmx) + m_use4;
        const float m_new = mx > m_run + kSlack ? mx : m_run;
        const float alpha = m_run == -__builtin_inff() ? 0.0f
                                                       : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        wfed *= alpha;
#pragma unroll
        for (int t = 0; t < T::NT; ++t) acc[t] *= alpha;
        m_run = m_new;
        const float mu = m_run == -__builtin_inff() ? 0.0f : m_run;
        const float d = m_use4 - mu;
        for (auto& x : sv) x += d;
        m_use4 = mu;
        sinit = -(cq + mu);
        thr4 = m_run == -__builtin_inff() ? -__builtin_inff() : kSlack;
    };

    auto consume = [&](int s, int i, bool refill) {
        if ((i >> 6) != batchA) {   // the consumer enters the next batch
            A = Bm;
            ++batchA;
            if ((batchA + 1) * 64 < cnt) Bm = load_meta(batchA + 1);
        }
        const int info = cur_info(i);
        const uint32_t mask = cur_mask(i);
        const bool seg_first = (info >> 5) & 1;
        const bool seg_last = (info >> 6) & 1;
        const int seg = (int)((unsigned)info >> 8);
        if (seg_first || i == 0) piece_start(seg, seg_first);
        // 4-bit value scales of this block, taken before the slot is refilled
        const f32x4 vsb = I4 ? vsr[s] : f32x4{1.0f, 1.0f, 1.0f, 1.0f};
        const int pb_i = cur_id(i);
        // block scales, read while every lane is active (a readlane inside a
        // divergent branch would read an unselected lane's stale register)
        const float ksc = QUANT ? cur_f(A.ksc, i) : 1.0f;
        const float vsc = QUANT ? cur_f(A.vsc, i) : 1.0f;
        if (pb_i < 0) piece_bad = true;
        if (!I4 && a.k_new != nullptr && seg_last && pb_i >= 0) {
            // fused decode step: this block holds the row's newest position
            // n - 1; its K/V rows come from the new token (replacing what
            // the tile load brought) and are written to the cache slot
            const int b = seg / n_kv, j = seg - (seg / n_kv) * n_kv;
            const int r = (nn[b] - 1) & 15;
            char* kt = (char*)kbase + (int64_t)pb_i * block_stride + (int64_t)j * head_stride;
            char* vt = (char*)vbase + (int64_t)pb_i * block_stride + (int64_t)j * head_stride;
            // the prefetched rows into this wave's LDS buffer as cache
            // codes (8-bit caches: each lane encodes the elements it holds),
            // where the lanes that hold row r of the tile read their pieces
            if (8 * lane < new_rowb) {
                if constexpr (QUANT) {
                    const int per = a.new_dtype == DT_F32 ? 2 : 4;   // elements per lane
                    const uint32_t ck = encode_lane<KV>(nkr[s], a.new_dtype, __fdiv_rn(1.0f, ksc));
                    const uint32_t cv = encode_lane<KV>(nvr[s], a.new_dtype, __fdiv_rn(1.0f, vsc));
                    if (per == 4) {
                        *(uint32_t*)(newk + 4 * lane) = ck;
                        *(uint32_t*)(newv + 4 * lane) = cv;
                    } else {
                        *(uint16_t*)(newk + 2 * lane) = (uint16_t)ck;
                        *(uint16_t*)(newv + 2 * lane) = (uint16_t)cv;
                    }
                } else {
                    *(uint2*)(newk + 8 * lane) = nkr[s];
                    *(uint2*)(newv + 8 * lane) = nvr[s];
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the writes have landed
            __builtin_amdgcn_wave_barrier();
            // newk / newv now hold row r in the cache's own bytes
            if constexpr (KST) {
#pragma unroll
                for (int l = 0; l < T::LOADS; ++l) {
                    if (vrow[l] == r) {   // contiguous K: same lanes as V
                        const int b0 = (1024 * l + 16 * lane) - r * T::ROWB;
                        const uint4 w = *(const uint4*)(newk + b0);
                        kr[s][l] = w;
                        *(uint4*)(kt + 1024 * l + 16 * lane) = w;
                    }
                }
            } else if (col == r) {
#pragma unroll
                for (int l = 0; l < T::LOADS; ++l) {
                    const uint4 w = *(const uint4*)(newk + 64 * l + 16 * grp);
                    kr[s][l] = w;
                    *(uint4*)(kt + r * T::ROWB + 64 * l + 16 * grp) = w;
                }
            }
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l) {
                if (vrow[l] == r) {
                    const uint4 w = *(const uint4*)(newv + (1024 * l + 16 * lane) - r * T::ROWB);
                    vr[s][l] = w;
                    *(uint4*)(vt + 1024 * l + 16 * lane) = w;
                }
            }
        }
        if (!I4 && mask != 0xFFFFu) {
            // rows past the sequence's end (or outside the window) may hold
            // stale data, possibly NaN: zero them so 0-weight products stay 0
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l)
                if (!((mask >> vrow[l]) & 1u)) vr[s][l] = make_uint4(0, 0, 0, 0);
        }
        // stage V (as bf16) into this wave's LDS tile
        if constexpr (I4) {
            // lane (t, grp): token row t, channels (d_h / 4) grp .. in groups of 8
            const uint32_t vw[4] = {vr[s][0].x, vr[s][0].y, vr[s][0].z, vr[s][0].w};
#pragma unroll
            for (int c = 0; c < T::LB / 4; ++c)
                *(bf16x8*)(stage + lds_off<HD>(col, (HD / 32) * grp + c)) =
                    int4x8_to_bf16_biased(vw[c]);
        }
#pragma unroll
        for (int l = 0; l < (I4 ? 0 : T::LOADS); ++l) {
            if (KV == DT_BF16) {
                *(uint4*)(stage + lds_off<HD>(vrow[l], vcb[l])) = vr[s][l];
            } else {
                const bf16x8 v0 = kv_operand_from_bytes<KV>(vr[s][l], 0);
                const bf16x8 v1 = kv_operand_from_bytes<KV>(vr[s][l], 1);
                *(bf16x8*)(stage + lds_off<HD>(vrow[l], vcb[l])) = v0;
                *(bf16x8*)(stage + lds_off<HD>(vrow[l], vcb[l] + 1)) = v1;
            }
        }
        if constexpr (KST) {
            // K tile into LDS: row r's 16-B chunk c at chunk c ^ kswz(r), so
            // that both this write (a 16-lane group covers one 256-B row, or
            // two 128-B rows) and the operand read below (16 lanes: 16 rows,
            // one chunk each) are free of bank conflicts
#pragma unroll
            for (int l = 0; l < T::LOADS; ++l)
                *(uint4*)(kstage + vrow[l] * T::ROWB +
                          16 * ((lane % T::CPRB) ^ kswz<HD>(vrow[l]))) = kr[s][l];
        }
        // scores S^T = K . Q^T; with an fp32 query the hi and lo passes go
        // to separate accumulators, two independent chains of matrix
        // products (4-bit: one chain from sinit, in the log2 domain)
        f32x4 st = {0, 0, 0, 0}, stl = {0, 0, 0, 0};
        if constexpr (I4) st = f32x4{sinit, sinit, sinit, sinit};
#pragma unroll
        for (int c = 0; c < T::NCH; ++c) {
            bf16x8 kop;
            if constexpr (KST) {
                kop = *(const bf16x8*)(kstage + col * T::ROWB + 16 * ((4 * c + grp) ^ kswz<HD>(col)));
            } else if constexpr (I4) {
                const uint32_t kw[4] = {kr[s][0].x, kr[s][0].y, kr[s][0].z, kr[s][0].w};
                kop = int4x8_to_bf16_biased(kw[c]);
            } else {
                kop = kv_operand_from_bytes<KV>(kr[s][c / 2], c % 2);
            }
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qhi[c], st, 0, 0, 0);
            if constexpr (I4)
                st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qlo[c], st, 0, 0, 0);
            else if (QT == DT_F32)
                stl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qlo[c], stl, 0, 0, 0);
        }
        if (QT == DT_F32 && !I4) st += stl;
        // refill this slot with the block kDepth ahead
        if (refill) issue(s, i + kDepth);

        // online softmax over this block's 16 tokens (base-2 domain)
        const float mult = a.scale_log2 * ksc;
        float sv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[e] = I4 ? st[e] : st[e] * mult;
        if (mask != 0xFFFFu) {   // wave-uniform: a partial or windowed block
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!((mask >> (4 * grp + e)) & 1u)) sv[e] = -__builtin_inff();
        }
        const float lmx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        // Lazy rescaling: the reference max of a head moves only when the
        // block's max exceeds it by more than kSlack (log2 units), so the
        // weights stay below 2^kSlack and the accumulators are rescaled in
        // the rare blocks where some head's max jumps (the first block of a
        // piece always sets it). Any reference gives the same softmax: the
        // partial carries (reference, sum) together.
        if (I4 && __builtin_amdgcn_ballot_w64(lmx > thr4) != 0) {
            rescale4(lmx, sv);
        } else if (!I4 && __builtin_amdgcn_ballot_w64(lmx > m_run + kSlack) != 0) {
            // some head's block max exceeds its reference by more than the
            // slack (a head's max exceeds iff one of its four lanes' does):
            // only then is the cross-lane max of each head formed
            const float mx = max_rows4(lmx);
            const float m_new = mx > m_run + kSlack ? mx : m_run;
            const float alpha = m_run == -__builtin_inff() ? 0.0f
                                                           : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < T::NT; ++t) acc[t] *= alpha;
            m_run = m_new;
        }
        const float m_use = (I4 || m_run == -__builtin_inff()) ? 0.0f : m_run;
        float pe[4], psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pe[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
            psum += pe[e];
        }
        l_run += psum;

        float pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pw[e] = pe[e] * (I4 ? vsb[e] : vsc);
        if (I4 && mask != 0xFFFFu) {   // the pad block: its scales may be anything
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!((mask >> (4 * grp + e)) & 1u)) pw[e] = 0.0f;
        }
        const bf16x8 pop = pack_p(pw);
        if constexpr (I4) {
            const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
            wfed = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), pop,
                                                           wfed, 0, 0, 0);
        }

        // O^T += [V^T | V^T] . [P_hi ; P_lo]
#pragma unroll
        for (int t = 0; t < T::NT; ++t) {
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)trd0[t]);
            const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)trd1[t]);
            const s16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pop,
                                                              acc[t], 0, 0, 0);
        }
        if (seg_last || i == cnt - 1) flush(seg, piece_whole && seg_last && !((info >> 4) & 1));
    };

    // 4-bit cache, steady state: blocks i and i + 1 (slots s and s + 1) of
    // one piece in one online-softmax step -- two independent chains of
    // score and value products per wave, and the step's control (maximum,
    // rescale test, sums) paid once per 32 tokens. Segments have even block
    // counts and ranges are cut between pairs, so i is even within its
    // segment and both blocks belong to the same piece; block i is a full
    // block, block i + 1 full or the segment's masked pad.
    auto consume_pair = [&](int s, int i) {
        enter(i);
        const int info0 = cur_info(i);
        const int pb0 = cur_id(i);
        enter(i + 1);
        const int info1 = cur_info(i + 1);
        const int pb1 = cur_id(i + 1);
        const uint32_t mask1 = cur_mask(i + 1);   // 0 for the pad block, else full
        const bool seg_first = (info0 >> 5) & 1;
        const bool seg_last = (info1 >> 6) & 1;
        const int seg = (int)((unsigned)info0 >> 8);
        if (seg_first || i == 0) piece_start(seg, seg_first);
        const f32x4 vsb0 = vsr[s], vsb1 = vsr[s + 1];
        if (pb0 < 0 || pb1 < 0) piece_bad = true;
        // both V tiles into this wave's two LDS tiles
        {
            const uint32_t w0[4] = {vr[s][0].x, vr[s][0].y, vr[s][0].z, vr[s][0].w};
            const uint32_t w1[4] = {vr[s + 1][0].x, vr[s + 1][0].y, vr[s + 1][0].z,
                                    vr[s + 1][0].w};
#pragma unroll
            for (int c = 0; c < T::LB / 4; ++c) {
                char* dst = stage + lds_off<HD>(col, (HD / 32) * grp + c);
                *(bf16x8*)dst = int4x8_to_bf16_biased(w0[c]);
                *(bf16x8*)(dst + kStage2) = int4x8_to_bf16_biased(w1[c]);
            }
        }
        // scores of both blocks: two independent chains (the hi and lo
        // query passes of each block accumulate together, from sinit)
        f32x4 s0 = {sinit, sinit, sinit, sinit}, s1 = s0;
        {
            const uint32_t k0[4] = {kr[s][0].x, kr[s][0].y, kr[s][0].z, kr[s][0].w};
            const uint32_t k1[4] = {kr[s + 1][0].x, kr[s + 1][0].y, kr[s + 1][0].z,
                                    kr[s + 1][0].w};
#pragma unroll
            for (int c = 0; c < T::NCH; ++c) {
                const bf16x8 a0 = int4x8_to_bf16_biased(k0[c]);
                const bf16x8 a1 = int4x8_to_bf16_biased(k1[c]);
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qhi[c], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qhi[c], s1, 0, 0, 0);
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qlo[c], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qlo[c], s1, 0, 0, 0);
            }
        }
        issue(s, i + kDepth);
        issue(s + 1, i + 1 + kDepth);

        // online softmax over the step's 32 tokens (base-2 domain, relative
        // to m_use4)
        float sv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sv[e] = s0[e];
            sv[4 + e] = mask1 != 0 ? s1[e] : -__builtin_inff();
        }
        // the NaN-propagating maximum takes matrix-product results as they
        // are (fmaxf would first quiet each one with an extra instruction);
        // a NaN score (from a NaN query) makes the output NaN either way
        auto mx3 = [](float x, float y, float z) {
            return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
        };
        const float lmx = mx3(mx3(sv[0], sv[1], sv[2]), mx3(sv[3], sv[4], sv[5]),
                              __builtin_elementwise_maximum(sv[6], sv[7]));
        if (__builtin_amdgcn_ballot_w64(lmx > thr4) != 0) rescale4(lmx, sv);
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(sv[e]);
        l_run += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
        float w0[4], w1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w0[e] = pe[e] * vsb0[e];
            w1[e] = mask1 != 0 ? pe[4 + e] * vsb1[e] : 0.0f;
        }
        const bf16x8 p0 = pack_p(w0), p1 = pack_p(w1);
        const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        wfed = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), p0, wfed,
                                                       0, 0, 0);
        wfed = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), p1, wfed,
                                                       0, 0, 0);
        // O^T += [V0^T | V0^T] . [P0_hi ; P0_lo] + [V1^T | V1^T] . [P1_hi ; P1_lo].
        // The empty asm redefines each address register in place once per
        // step, so the second tile's address (kStage2 past the first) cannot
        // be hoisted into registers of its own and is folded into the read's
        // offset instead.
#pragma unroll
        for (int t = 0; t < T::NT; ++t) asm volatile("" : "+v"(trd0[t]), "+v"(trd1[t]));
#pragma unroll
        for (int t = 0; t < T::NT; ++t) {
            const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)trd0[t]);
            const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)trd1[t]);
            const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(uintptr_t)(trd0[t] + kStage2));
            const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(uintptr_t)(trd1[t] + kStage2));
            const s16x8 va = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const s16x8 vb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), p0,
                                                              acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vb), p1,
                                                              acc[t], 0, 0, 0);
        }
        if (seg_last || i + 1 == cnt - 1)
            flush(seg, piece_whole && seg_last && !((info1 >> 4) & 1));
    };

    // the first segment's queries, in flight with the first tiles (4-bit:
    // fetched before them, combined after them)
    q_seg = (int)((unsigned)meta_info(0) >> 8);
    if constexpr (I4) q_fetch(q_seg);
    else load_q(q_seg);
    __builtin_amdgcn_sched_barrier(0);
    int it = 0;
    if (cnt >= 2 * kDepth) {
        // prologue and steady state issue unconditionally and in slot order
        // (the scheduling barriers keep the prologue's independent loads from
        // being reordered), so at the loop head the newest loads are always
        // the other slots' and each block waits only for itself
#pragma unroll
        for (int s = 0; s < kDepth; ++s) {
            issue(s, s);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (I4) load_q(q_seg, true);
        for (; it + 2 * kDepth <= cnt; it += kDepth) {
            if constexpr (I4) {
                static_assert(kDepth % 2 == 0, "4-bit steps take blocks in pairs");
#pragma unroll
                for (int s = 0; s < kDepth; s += 2) consume_pair(s, it + s);
            } else {
#pragma unroll
                for (int s = 0; s < kDepth; ++s) consume(s, it + s, true);
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < kDepth; ++s)
            if (s < cnt) issue(s, s);
        if constexpr (I4) load_q(q_seg, true);
    }
    // drain: fewer than 2 * kDepth blocks remain, their first loads issued
#pragma unroll
    for (int k = 0; k < 2 * kDepth; ++k)
        if (it + k < cnt) consume(k % kDepth, it + k, it + k + kDepth < cnt);
}

}  // namespace

// pre, nn and preu, plus the prefix lengths for the shared-prefix calls
size_t attn_mfma_dyn_lds(int32_t B, bool prefix) {
    return (size_t)((prefix ? 4 : 3) * B + 2) * sizeof(int32_t);
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
    const int waves = a.split ? a.nw : a.B * a.n_kv;
    dim3 grid((waves + 3) / 4);
    dim3 block(kAttnThreads);
    const size_t lds = attn_mfma_dyn_lds(a.B, a.prefix_lens != nullptr);
#define PDA_LAUNCH(HD, KV, QT) \
    hipLaunchKernelGGL((k_attn_mfma<HD, KV, QT>), grid, block, lds, s, a)
#define PDA_BY_Q(HD, KV)                          \
    if (a.q_dtype == DT_BF16) PDA_LAUNCH(HD, KV, DT_BF16); \
    else PDA_LAUNCH(HD, KV, DT_F32)
#define PDA_BY_KV(HD)                                         \
    if (a.kv_dtype == DT_BF16) { PDA_BY_Q(HD, DT_BF16); }     \
    else if (a.kv_dtype == DT_FP8) { PDA_BY_Q(HD, DT_FP8); }  \
    else if (a.kv_dtype == DT_INT8) { PDA_BY_Q(HD, DT_INT8); } \
    else { PDA_BY_Q(HD, DT_INT4); }
    if (a.d_h == 128) { PDA_BY_KV(128); }
    else { PDA_BY_KV(64); }
#undef PDA_BY_KV
#undef PDA_BY_Q
#undef PDA_LAUNCH
    return hipGetLastError();
}

}  // namespace pda
