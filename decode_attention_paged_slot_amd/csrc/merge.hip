// merge.hip -- log-sum-exp merge of split-KV partial results.
//
// A partition's partial is (o_p, m_p, l_p): its output normalised over its own
// tokens, the max of its base-2 scores and the sum of 2^(score - m_p). Since
// softmax over the union is sum_p l_p 2^(m_p - M) o_p / sum_p l_p 2^(m_p - M)
// with M = max_p m_p, partials merge exactly; empty partials (l_p = 0) drop
// out. The split keeps the single cache read and the no-score-spill property
// of the attention step (SoK paper appendices A.1, C.4).
//
// Two forms. Rows with few pieces and no residual-window piece: one wave per
// output row, every load in flight at once, wave reductions only
// (k_merge_rows). Otherwise one workgroup per output row (or per column
// slice of it): a block-wide max and sum over the partials' statistics, then
// a weighted sum of the partial outputs split over partition subsets,
// combined through LDS (merge_row).
#include "device_common.h"
#include "pda_internal.h"

namespace pda {

namespace {

constexpr int kThreads = 256;
constexpr int kMergeColumnSplit = 4;   // workgroups per output row when segments have many pieces

// Block-wide max and sum of a 4-wave workgroup. Each takes its own 4-float
// LDS slot (`red`) and is used once per workgroup, so no barrier is needed
// after the slot is read.
__device__ __forceinline__ float block_max(float v, float* red) {
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float v, float* red) {
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Merge of the partials of one output row into `out_row` (HD floats or
// bf16), columns [c0 * 4, (c0 + V) * 4) of it. The partials come from two
// strided runs: p < n1 has statistics (m, l) at ml1 + p * sm1 and output at
// po1 + p * so1, p = n1 + k (k < n2) at ml2 + k * sm2 and po2 + k * so2.
// Phase 1: every thread takes partials p = tid, tid + 256, ... for the
// block-wide max M and the weights w_p = l_p 2^(m_p - M), kept in LDS.
// Phase 2: thread (sub, c) accumulates the 4-float column group c0 + c of
// the partials p = sub, sub + SUB, ... (loads are unconditional, so they can
// all be in flight together; an empty partial's weight is 0 and its data
// unused); the SUB partial sums are added through LDS.
struct PieceRuns {
    const float* po1;
    const float* ml1;
    int64_t so1, sm1;
    int n1;
    const float* po2;
    const float* ml2;
    int64_t so2, sm2;
    int n2;
    __device__ __forceinline__ const float* ml(int p) const {
        return p < n1 ? ml1 + p * sm1 : ml2 + (p - n1) * sm2;
    }
    __device__ __forceinline__ const float* po(int p) const {
        return p < n1 ? po1 + p * so1 : po2 + (p - n1) * so2;
    }
};

// An extra piece (xm, xl, xo) formed by the workgroup itself joins when
// xl != 0: xm, xl are its statistics (the same in every thread) and xo this
// thread's share of its unnormalised output sum_t 2^(s_t - xm) v_t over the
// tokens of the thread's subset, for its column group; it enters with weight
// xl 2^(xm - M) and output contribution 2^(xm - M) xo. `extra(xm, xl, xo)`
// forms it (every thread calls it); it runs after the first partial outputs
// and statistics have been requested, so its own loads share their round
// trip.
struct NoExtraPiece {
    __device__ __forceinline__ void operator()(float& xm, float& xl, f32x4& xo) const {
        xm = -__builtin_inff();
        xl = 0.0f;
        xo = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
};

template <int V, class Extra>
__device__ __forceinline__ void merge_row(const PieceRuns& pr, bool row_bad, int c0,
                                          void* out_row, int32_t out_dtype, float* wsh,
                                          float* red, f32x4* acc_sh, Extra extra) {
    constexpr int SUB = kThreads / V;  // partial subsets
    constexpr int KP = 4;              // partial outputs loaded ahead per thread
    const int np = pr.n1 + pr.n2;
    const int c = threadIdx.x % V, sub = threadIdx.x / V;
    // The first KP partial outputs of this thread are loaded before the
    // statistics are reduced, so the two phases share one memory round trip
    // (a row has few pieces: most rows finish with these).
    f32x4 ov[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int p = min(sub + k * SUB, np - 1);
        ov[k] = np > 0 ? *((const f32x4*)pr.po(p) + c0 + c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // this thread's first statistics (piece threadIdx.x), in flight with them
    const bool has0 = (int)threadIdx.x < np;
    const float2 x0 = has0 ? *(const float2*)pr.ml(threadIdx.x) : make_float2(0.0f, 0.0f);
    float xm, xl;
    f32x4 xo;
    extra(xm, xl, xo);
    float mloc = xl != 0.0f ? xm : -__builtin_inff();
    if (has0 && x0.y != 0.0f) mloc = fmaxf(mloc, x0.x);
    for (int p = threadIdx.x + kThreads; p < np; p += kThreads) {
        const float2 x = *(const float2*)pr.ml(p);
        if (x.y != 0.0f) mloc = fmaxf(mloc, x.x);
    }
    const float M = block_max(mloc, red);   // red[0..3]
    const float xs = xl != 0.0f ? __builtin_amdgcn_exp2f(xm - M) : 0.0f;
    float lsum = threadIdx.x == 0 ? xl * xs : 0.0f;
    if (has0) {
        const float w = x0.y == 0.0f ? 0.0f : x0.y * __builtin_amdgcn_exp2f(x0.x - M);
        wsh[threadIdx.x] = w;
        lsum += w;
    }
    for (int p = threadIdx.x + kThreads; p < np; p += kThreads) {
        const float2 x = *(const float2*)pr.ml(p);
        const float w = x.y == 0.0f ? 0.0f : x.y * __builtin_amdgcn_exp2f(x.x - M);
        wsh[p] = w;
        lsum += w;
    }
    const float L = block_sum(lsum, red + 4);   // its barrier also publishes wsh
    f32x4 acc = xs * xo;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int p = sub + k * SUB;
        if (p < np) {
            const float w = wsh[p];
            if (w != 0.0f) acc += w * ov[k];
        }
    }
#pragma unroll 4
    for (int p = sub + KP * SUB; p < np; p += SUB) {
        const f32x4 o = *((const f32x4*)pr.po(p) + c0 + c);
        const float w = wsh[p];
        if (w != 0.0f) acc += w * o;
    }
    // the SUB subset sums of a column: within a wave they sit in lanes c,
    // c + V, ... and add by lane exchanges; the four waves' sums meet in LDS
    static_assert(64 % V == 0 && kThreads == 256, "column groups tile a wave");
#pragma unroll
    for (int o = V; o < 64; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o, 64);
        acc.y += __shfl_xor(acc.y, o, 64);
        acc.z += __shfl_xor(acc.z, o, 64);
        acc.w += __shfl_xor(acc.w, o, 64);
    }
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) < V) acc_sh[wv * V + c] = acc;
    __syncthreads();
    if (sub == 0) {
        const f32x4 tot = (acc_sh[c] + acc_sh[V + c]) + (acc_sh[2 * V + c] + acc_sh[3 * V + c]);
        f32x4 r;
        const bool ok = L != 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = ok ? tot[e] / L : 0.0f;
        if (row_bad) r = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                               __builtin_nanf("")};
        if (out_dtype == DT_F32) {
            *((f32x4*)out_row + c0 + c) = r;
        } else {
            uint2 h;
            h.x = f32_to_bf16_rne(r[0]) | (f32_to_bf16_rne(r[1]) << 16);
            h.y = f32_to_bf16_rne(r[2]) | (f32_to_bf16_rne(r[3]) << 16);
            *((uint2*)out_row + c0 + c) = h;
        }
    }
}

// Partition layout (rows x P partials). context_lens != nullptr: row r
// belongs to sequence r / n_q and uses the partitions its length needs
// (ceil(ceil(n / 16) / bpp), capped at P); otherwise all P partials are read
// and l_p == 0 marks an empty one.
template <int HD>
__global__ void __launch_bounds__(kThreads) k_merge(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    const int32_t* __restrict__ context_lens,
                                                    int32_t n_q, int32_t P, int32_t bpp,
                                                    int32_t max_blocks, void* out,
                                                    int32_t out_dtype) {
    __shared__ float wsh[kMaxPartitions];
    __shared__ float red[8];   // block_max, block_sum
    __shared__ f32x4 acc_sh[kThreads];
    const int64_t row = blockIdx.x;
    int np = P;
    bool row_bad = false;
    if (context_lens) {
        const int n = context_lens[row / n_q];
        row_bad = n < 0 || n > max_blocks * 16;
        const int nblk = row_bad ? 0 : (n + 15) >> 4;
        np = min(P, (nblk + bpp - 1) / bpp);
    }
    char* orow = (char*)out + row * HD * (out_dtype == DT_F32 ? 4 : 2);
    const PieceRuns pr{part_o + row * (int64_t)P * HD, part_ml + row * (int64_t)P * 2, HD, 2, np,
                       nullptr, nullptr, 0, 0, 0};
    merge_row<HD / 4>(pr, row_bad, 0, orow, out_dtype, wsh, red, acc_sh, NoExtraPiece{});
}

// The residual window of a 4-bit cache as an extra piece of output row
// `row` = b * n_q + h (SoK paper section 2.3: the newest tokens stay at full
// precision until their group is quantized): its r = n % 16 newest tokens,
// bf16 rows of k_res / v_res [B][n_kv][16][d_h], j = h / g. Thread tid forms
// the partial dot product of q with k_t, t = tid / 16, over channels
// (tid % 16) * d_h / 16 .. +d_h / 16; a 16-lane reduction gives the base-2
// score s_t = scale * log2(e) * <q, k_t>, and the 16 scores pass through LDS
// so that every thread forms m = max_t s_t and l = sum_t 2^(s_t - m) in the
// same order. Thread (sub, c) then sums 2^(s_t - m) v_t over the tokens
// t = sub, sub + SUB, ... for its column group c0 + c.
template <int HD, int V>
__device__ __forceinline__ void residual_piece(const AttnArgs& a, int64_t row, int b, int j,
                                               int r, int c0, float* s_sh, float& xm,
                                               float& xl, f32x4& xo) {
    constexpr int SUB = kThreads / V;
    constexpr int TPS = (16 + SUB - 1) / SUB;   // tokens per subset
    constexpr int CP = HD / 16;                 // channels per thread in the scores
    const int tid = threadIdx.x;
    const int64_t rbase = ((int64_t)b * a.n_kv + j) * 16;   // residual rows of (b, j)
    const uint16_t* kres = (const uint16_t*)a.k_res;
    const uint16_t* vres = (const uint16_t*)a.v_res;
    const int c = tid % V, sub = tid / V;
    uint2 vw[TPS];
#pragma unroll
    for (int k = 0; k < TPS; ++k) {
        const int tt = sub + k * SUB;
        vw[k] = tt < r ? *(const uint2*)(vres + (rbase + tt) * HD + 4 * (c0 + c))
                       : make_uint2(0, 0);
    }
    const int t = tid >> 4, part = tid & 15;
    float dot = 0.0f;
    if (t < r) {
        float kf[CP], qf[CP];
        const uint16_t* kp = kres + (rbase + t) * HD + part * CP;
        if constexpr (CP == 8) {
            const uint4 w = *(const uint4*)kp;
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = bf16_lo_to_f32(ws[e]);
                kf[2 * e + 1] = bf16_hi_to_f32(ws[e]);
            }
        } else {
            const uint2 w = *(const uint2*)kp;
            kf[0] = bf16_lo_to_f32(w.x); kf[1] = bf16_hi_to_f32(w.x);
            kf[2] = bf16_lo_to_f32(w.y); kf[3] = bf16_hi_to_f32(w.y);
        }
        if (a.q_dtype == DT_BF16) {
            const uint16_t* qp = (const uint16_t*)a.q + row * HD + part * CP;
#pragma unroll
            for (int e = 0; e < CP; ++e) qf[e] = __uint_as_float((uint32_t)qp[e] << 16);
        } else {
            const float* qp = (const float*)a.q + row * HD + part * CP;
#pragma unroll
            for (int e = 0; e < CP; ++e) qf[e] = qp[e];
        }
#pragma unroll
        for (int e = 0; e < CP; ++e) dot += qf[e] * kf[e];
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) dot += __shfl_xor(dot, o, 64);
    if (part == 0) s_sh[t] = t < r ? dot * a.scale_log2 : -__builtin_inff();
    __syncthreads();
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < 16; ++k) m = fmaxf(m, s_sh[k]);
    float l = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) l += k < r ? __builtin_amdgcn_exp2f(s_sh[k] - m) : 0.0f;
    f32x4 o4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < TPS; ++k) {
        const int tt = sub + k * SUB;
        if (tt < r) {
            const float w = __builtin_amdgcn_exp2f(s_sh[tt] - m);
            o4[0] += w * bf16_lo_to_f32(vw[k].x);
            o4[1] += w * bf16_hi_to_f32(vw[k].x);
            o4[2] += w * bf16_lo_to_f32(vw[k].y);
            o4[3] += w * bf16_hi_to_f32(vw[k].y);
        }
    }
    xm = m;
    xl = l;
    xo = o4;
}

// Stream layout (attention kernel's split mode): output row r = seg * g + hh
// of segment seg; the pieces of a split segment sit in slots seg + w for the
// waves w in seg_info[seg] = (first, last), piece row (seg + w) * g + hh.
// Segments with a single piece (written by the attention kernel directly)
// or none (zero / NaN rows, also written there) are skipped. With a shared
// prefix (prefix_lens != nullptr), a row whose prefix has p blocks also has
// the prefix pass's pieces of chunks 0 .. ceil(p / kPrefixChunk) - 1, at row
// c * rows + r of pre_o / pre_ml, and its stream pieces always come here. A
// valid row of a 4-bit cache with n % 16 != 0 residual-window tokens has one
// more piece, formed here from its bf16 residual rows (residual_piece), and
// also always comes here.
// With CS > 1 workgroups per row (grid.y), workgroup (row, cs) handles the
// cs-th of CS column ranges, so rows with many pieces are spread over
// several compute units. The weights live in dynamic LDS sized for the wave
// count plus the prefix chunks.
template <int HD, int CS>
__global__ void __launch_bounds__(kThreads) k_merge_stream(AttnArgs a) {
    constexpr int V = HD / 4 / CS;
    extern __shared__ float wsh[];
    __shared__ float red[8];   // block_max, block_sum
    __shared__ f32x4 acc_sh[kThreads];
    __shared__ float s_sh[16];
    const int64_t row = blockIdx.x;
    const int g = a.g;
    const int64_t seg = row / g;
    const int hh = (int)(row - seg * g);
    const int2 info = a.seg_info[seg];
    const int np = info.y - info.x + 1;
    const int b = (int)(row / a.n_q);
    int npre = 0, r_res = 0;
    if (a.prefix_lens != nullptr) {
        const int pl = row_prefix_len(a.context_lens[b], a.prefix_lens[b], a.max_blocks,
                                      a.prefix_blocks);
        npre = pl > 0 ? (pl + kPrefixChunk - 1) / kPrefixChunk : 0;
    } else if (a.k_res != nullptr) {
        // the residual window of a valid row; an invalid row keeps the NaN
        // the attention kernel wrote
        const int n = a.context_lens[b];
        r_res = (n >= 0 && n <= a.max_blocks * 16) ? n % 16 : 0;
    }
    if (npre == 0 && r_res == 0 && np <= 1) return;
    const int c0 = (int)blockIdx.y * V;
    const int64_t prow0 = (seg + info.x) * g + hh;
    const int64_t rows = (int64_t)a.B * a.n_q;
    char* orow = (char*)a.out + row * HD * (a.out_dtype == DT_F32 ? 4 : 2);
    const PieceRuns pr{a.part_o + prow0 * HD, a.part_ml + prow0 * 2, (int64_t)g * HD,
                       (int64_t)g * 2, max(np, 0),
                       npre ? a.pre_o + row * HD : nullptr, npre ? a.pre_ml + row * 2 : nullptr,
                       rows * HD, rows * 2, npre};
    // the residual window's piece is formed once the stored pieces' loads
    // are in flight
    merge_row<V>(pr, false, c0, orow, a.out_dtype, wsh, red, acc_sh,
                 [&](float& xm, float& xl, f32x4& xo) {
                     NoExtraPiece{}(xm, xl, xo);
                     if (r_res > 0)
                         residual_piece<HD, V>(a, row, b, (int)(seg % a.n_kv), r_res, c0, s_sh,
                                               xm, xl, xo);
                 });
}

// Stream layout without a residual window and with few pieces per row: one
// wave per output row. A row's pieces are its stream pieces, then (with a
// shared prefix) the prefix pass's pieces of its prefix chunks. Pieces are
// taken in batches of up to 32: lane l holds the statistics of piece
// p0 + l, and the partial outputs of its float4 column c = l % C (C = d_h / 4
// columns) for pieces p0 + h, p0 + h + H, ... (h = l / C, H = 64 / C). All
// of a batch's loads are issued before any is used; the batch max and weight
// sum are wave reductions, a piece's weight reaches the lanes holding its
// output by a lane shuffle, and the H partial sums of a column meet by lane
// exchanges: no LDS, no barrier. A later batch rescales the running sums to
// the new max. As in merge_row, a piece with l_p = 0 drops out and a NaN l_p
// (a piece that met an unmapped block) makes the row NaN.
template <int HD>
__global__ void __launch_bounds__(kThreads) k_merge_rows(AttnArgs a) {
    constexpr int C = HD / 4;    // float4 columns of a row
    constexpr int H = 64 / C;    // lanes per column
    constexpr int KB = 32;       // pieces per batch
    constexpr int PL = KB / H;   // pieces per lane and batch
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= (int64_t)a.B * a.n_q) return;
    const int g = a.g;
    const int64_t seg = row / g;
    const int hh = (int)(row - seg * g);
    const int2 info = a.seg_info[seg];
    const int ns = max(info.y - info.x + 1, 0);   // stream pieces
    int npre = 0;                                 // prefix pieces
    if (a.prefix_lens != nullptr) {
        const int b = (int)(row / a.n_q);
        const int pl = row_prefix_len(a.context_lens[b], a.prefix_lens[b], a.max_blocks,
                                      a.prefix_blocks);
        npre = pl > 0 ? (pl + kPrefixChunk - 1) / kPrefixChunk : 0;
    }
    // without prefix pieces, a single piece was written to the output by the
    // attention kernel, and so were the zero / NaN rows of empty or invalid
    // sequences (no piece)
    if (npre == 0 && ns <= 1) return;
    const int np = ns + npre;
    const int64_t prow0 = (seg + info.x) * g + hh;   // stream piece p: piece row prow0 + p * g
    const int64_t rows = (int64_t)a.B * a.n_q;
    // piece p's partial output and statistics
    auto po = [&](int p) {
        return p < ns ? a.part_o + (prow0 + (int64_t)p * g) * HD
                      : a.pre_o + ((int64_t)(p - ns) * rows + row) * HD;
    };
    auto pm = [&](int p) {
        return p < ns ? a.part_ml + (prow0 + (int64_t)p * g) * 2
                      : a.pre_ml + ((int64_t)(p - ns) * rows + row) * 2;
    };
    const int c = lane % C, h = lane / C;
    float M = -__builtin_inff(), L = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int p0 = 0; p0 < np; p0 += KB) {
        const int nb = min(KB, np - p0);
        f32x4 ov[PL];
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const int p = h + H * k;
            ov[k] = p < nb ? *((const f32x4*)po(p0 + p) + c) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        float2 st = make_float2(0.0f, 0.0f);
        if (lane < nb) st = *(const float2*)pm(p0 + lane);
        float mb = st.y != 0.0f ? st.x : -__builtin_inff();
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mb = fmaxf(mb, __shfl_xor(mb, o, 64));
        const float Mn = fmaxf(M, mb);
        const float w = st.y == 0.0f ? 0.0f : st.y * __builtin_amdgcn_exp2f(st.x - Mn);
        float lb = w;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) lb += __shfl_xor(lb, o, 64);
        const float f = M == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
        acc *= f;
        L = L * f + lb;
        M = Mn;
#pragma unroll
        for (int k = 0; k < PL; ++k) {
            const float wk = __shfl(w, h + H * k, 64);
            if (wk != 0.0f) acc += wk * ov[k];
        }
    }
#pragma unroll
    for (int o = C; o < 64; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o, 64);
        acc.y += __shfl_xor(acc.y, o, 64);
        acc.z += __shfl_xor(acc.z, o, 64);
        acc.w += __shfl_xor(acc.w, o, 64);
    }
    if (h == 0) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = L != 0.0f ? acc[e] / L : 0.0f;
        if (a.out_dtype == DT_F32) {
            *((f32x4*)((float*)a.out + row * HD) + c) = r;
        } else {
            uint2 o2;
            o2.x = f32_to_bf16_rne(r[0]) | (f32_to_bf16_rne(r[1]) << 16);
            o2.y = f32_to_bf16_rne(r[2]) | (f32_to_bf16_rne(r[3]) << 16);
            *((uint2*)((uint16_t*)a.out + row * HD) + c) = o2;
        }
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

hipError_t launch_merge_stream(const AttnArgs& a, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.n_q;
    if (rows == 0) return hipSuccess;
    const int chunks = a.prefix_blocks > 0 ? (a.prefix_blocks + kPrefixChunk - 1) / kPrefixChunk
                                           : 0;
    const size_t lds = (size_t)(a.nw + chunks) * sizeof(float);
    // split a row's columns over several workgroups only when segments
    // average many pieces (long sequences in a small batch)
    const bool wide = (int64_t)a.nw >= 64 * (int64_t)a.B * a.n_kv;
    if (!wide && a.k_res == nullptr) {
        // few pieces per row (stream and prefix pieces): one wave per row. (Rows with many
        // pieces keep the block-wide merge: split over column slices, waves
        // per row measured slower there, with fewer loads in flight.)
        const dim3 grid((unsigned)((rows + kThreads / 64 - 1) / (kThreads / 64)));
        if (a.d_h == 128) hipLaunchKernelGGL((k_merge_rows<128>), grid, dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((k_merge_rows<64>), grid, dim3(kThreads), 0, s, a);
        return hipGetLastError();
    }
#define PDA_MS(HD, CS)                                                                       \
    hipLaunchKernelGGL((k_merge_stream<HD, CS>), dim3(rows, CS), dim3(kThreads), lds, s, a)
    if (a.d_h == 128) {
        if (wide) PDA_MS(128, kMergeColumnSplit);
        else PDA_MS(128, 1);
    } else {
        if (wide) PDA_MS(64, kMergeColumnSplit);
        else PDA_MS(64, 1);
    }
#undef PDA_MS
    return hipGetLastError();
}

hipError_t launch_lse_merge(const float* part_o, const float* part_ml, int32_t rows, int32_t P,
                            int32_t d_h, float* out, hipStream_t s) {
    return launch_merge(part_o, part_ml, nullptr, rows, 1, P, 1, 0, d_h, out, DT_F32, s);
}

}  // namespace pda
