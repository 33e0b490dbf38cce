// api.cpp -- the C ABI: argument validation, split planning and dispatch.
// Every device call is one or two kernel launches on the caller's stream.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include <hip/hip_runtime.h>

#include "pda.h"
#include "pda_internal.h"

namespace pda {

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

thread_local char g_err[512] = "";

namespace {
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int32_t hip_fail(const char* what, hipError_t e) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return PDA_EHIP;
}

bool debug_mode() {
    const char* v = std::getenv("PDA_DEBUG");
    return v && v[0] && std::strcmp(v, "0") != 0;
}

int env_int(const char* name, int dflt) {
    const char* v = std::getenv(name);
    if (!v || !v[0]) return dflt;
    return std::atoi(v);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }
}  // namespace

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

// Partition plan (fp32 caches). The grid is (P, n_kv, B) with one workgroup
// of 4 waves per cell serving the g query heads of its KV head; aim at ~2048
// workgroups with 32..256 blocks per partition, so every wave streams at
// least 8 blocks and the partial results stay below 1% of the cache bytes.
Plan make_partition_plan(const pda_attn_desc& d) {
    const int64_t max_ctx = std::max<int64_t>(d.max_context, 1);
    const int32_t nblk_max =
        (int32_t)std::min<int64_t>(ceil_div(max_ctx, d.block_size), d.max_blocks_per_seq);
    Plan p{1, std::max(nblk_max, 1), 0, 0, 0};
    if (d.num_partitions == 1 || nblk_max <= 1) return p;
    int32_t bpp;
    if (d.num_partitions > 1) {
        bpp = ceil_div(nblk_max, d.num_partitions);
    } else {
        const int64_t ctx_blocks = d.total_context > 0 ? ceil_div(d.total_context, d.block_size)
                                                       : (int64_t)d.B * nblk_max;
        const int64_t tiles = ctx_blocks * d.n_kv;
        bpp = ceil_div(tiles, 2048);
        bpp = std::max(bpp, 32);
        bpp = std::min(bpp, 256);
        bpp = (bpp + 3) & ~3;
    }
    bpp = std::max(bpp, ceil_div(nblk_max, kMaxPartitions));
    p.bpp = std::max(bpp, 1);
    p.P = ceil_div(nblk_max, p.bpp);
    if (p.P <= 1) p = Plan{1, std::max(nblk_max, 1), 0, 0, 0};
    return p;
}

Plan make_stream_plan_split(const pda_attn_desc& d, int64_t S, int64_t t_est);

// Stream plan (16-bit and 8-bit caches). Measured on MI355X: the step runs
// at its best when every compute unit holds the same amount of work, and one
// workgroup of four streaming waves per compute unit already saturates HBM
// with a bf16 cache; so the default is one workgroup per compute unit of the
// current device (256 on an MI355X: 1024 wave ranges) for bf16 and two for
// 8-bit caches, fewer when the batch has under 8 blocks per range. One more
// workgroup than the device runs at once costs ~60% (the equal ranges then
// wait on a second round). The block count T is estimated from the
// host hints (total_context, else B * max_context); the kernel recomputes the
// exact split from context_lens, so the estimate only tunes the wave count.
Plan make_stream_plan(const pda_attn_desc& d) {
    const int64_t S = (int64_t)d.B * d.n_kv;
    const int64_t nblk_max = std::min<int64_t>(
        ceil_div(std::max<int64_t>(d.max_context, 1), d.block_size), d.max_blocks_per_seq);
    const int64_t t_est = (int64_t)d.n_kv *
        (d.total_context > 0 ? ceil_div(d.total_context, d.block_size) + d.B : d.B * nblk_max);
    Plan p{1, (int32_t)std::max<int64_t>(nblk_max, 1), (int32_t)S, 0, 1};
    if (d.prefix_blocks > 0 || d.kv_dtype == PDA_INT4) {
        // with a shared prefix (or a 4-bit cache's residual window) every
        // row's pieces go through the merge, so
        // the split bookkeeping is always on; "unsplit" is one range per segment
        Plan q = p;
        if (d.num_partitions != 1) q = make_stream_plan_split(d, S, t_est);
        if (!q.split) {
            q.nw = (int32_t)std::min<int64_t>(std::max<int64_t>(S, 1), kMaxStreamWaves);
            q.split = 1;
            q.P = q.nw;
            q.bpp = (int32_t)std::max<int64_t>(1, (t_est + q.nw - 1) / q.nw);
        }
        return q;
    }
    if (d.num_partitions == 1) return p;
    return make_stream_plan_split(d, S, t_est);
}

// Compute units of the current device, cached per device ordinal; 256 (an
// MI355X, one partition) when no device is current or the query fails. The
// streaming kernel's equal wave ranges assume that all of its workgroups run
// at once, so the default workgroup count follows the device's CU count
// (a partitioned GPU exposes fewer CUs per device).
int64_t device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// The split part of the stream plan (see make_stream_plan).
Plan make_stream_plan_split(const pda_attn_desc& d, int64_t S, int64_t t_est) {
    const int64_t nblk_max = std::min<int64_t>(
        ceil_div(std::max<int64_t>(d.max_context, 1), d.block_size), d.max_blocks_per_seq);
    Plan p{1, (int32_t)std::max<int64_t>(nblk_max, 1), (int32_t)S, 0, 1};
    int64_t nw;
    if (d.num_partitions > 1) {
        nw = d.num_partitions;
    } else {
        // one workgroup per compute unit; 8-bit caches do twice the
        // conversion and matrix work per byte and need two per compute unit
        // to keep HBM busy
        const bool eight_bit = d.kv_dtype == PDA_FP8_E4M3 || d.kv_dtype == PDA_INT8 ||
                               d.kv_dtype == PDA_INT4;
        const int64_t cus = device_cus();
        const int64_t wgs = std::max<int64_t>(
            env_int("PDA_ATTN_WORKGROUPS", (int)(eight_bit ? 2 * cus : cus)), 1);
        const int64_t min_blocks = std::max(env_int("PDA_MIN_BLOCKS_PER_WAVE", 8), 1);
        nw = std::min<int64_t>(4 * wgs, (t_est + min_blocks - 1) / min_blocks);
        // short contexts (a few blocks per segment): one wave per segment, no merge
        if (nw <= S && t_est <= S * 4 * min_blocks) return p;
    }
    nw = std::min<int64_t>(nw, kMaxStreamWaves);
    p.nw = (int32_t)nw;
    p.split = 1;
    p.P = (int32_t)nw;
    p.bpp = (int32_t)std::max<int64_t>(1, (t_est + nw - 1) / nw);
    return p;
}

Plan make_plan(const pda_attn_desc& d) {
    return d.kv_dtype == PDA_F32 ? make_partition_plan(d) : make_stream_plan(d);
}

WsLayout ws_layout(const pda_attn_desc& d, const Plan& p) {
    WsLayout w{0, 0, 0, 0, 0, 0};
    if (p.stream) {
        if (!p.split) return w;
        const size_t S = (size_t)d.B * d.n_kv;
        const size_t g = (size_t)(d.n_q / d.n_kv);
        const size_t slots = S + (size_t)p.nw;
        w.part_o_off = 0;
        w.part_ml_off = align256(slots * g * d.d_h * sizeof(float));
        w.seg_info_off = w.part_ml_off + align256(slots * g * 2 * sizeof(float));
        w.bytes = w.seg_info_off + align256(S * 2 * sizeof(int32_t));
        if (d.prefix_blocks > 0) {
            // prefix pass pieces
            const size_t chunks = (size_t)ceil_div(d.prefix_blocks, kPrefixChunk);
            const size_t rows = (size_t)d.B * d.n_q;
            w.pre_o_off = w.bytes;
            w.pre_ml_off = w.pre_o_off + align256(chunks * rows * d.d_h * sizeof(float));
            w.bytes = w.pre_ml_off + align256(chunks * rows * 2 * sizeof(float));
        }
        return w;
    }
    if (p.P <= 1) return w;
    const size_t rows = (size_t)d.B * d.n_q;
    w.part_o_off = 0;
    w.part_ml_off = align256(rows * p.P * d.d_h * sizeof(float));
    w.bytes = w.part_ml_off + align256(rows * p.P * 2 * sizeof(float));
    return w;
}

}  // namespace pda

using namespace pda;

namespace {

// Which call a descriptor is checked for.
enum CallKind { kPlain, kQuant, kPrefix, kInt4, kQuery };

int32_t check_attn_desc(const pda_attn_desc* d, CallKind kind) {
    if (!d) {
        set_error("attention descriptor is NULL");
        return PDA_EINVAL;
    }
    if (d->B < 0 || d->n_q <= 0 || d->n_kv <= 0 || d->n_q % d->n_kv != 0) {
        set_error("bad head counts: B=%d n_q=%d n_kv=%d", d->B, d->n_q, d->n_kv);
        return PDA_EINVAL;
    }
    const int g = d->n_q / d->n_kv;
    if (g > 16) {
        set_error("group factor %d > 16 unsupported", g);
        return PDA_EINVAL;
    }
    if (d->d_h != 64 && d->d_h != 128) {
        set_error("d_h=%d unsupported (64 or 128)", d->d_h);
        return PDA_EINVAL;
    }
    if (d->block_size != kBlockSize) {
        set_error("block_size=%d unsupported (16)", d->block_size);
        return PDA_EINVAL;
    }
    if (d->max_blocks_per_seq <= 0 || d->num_blocks <= 0 || d->max_context < 0 ||
        d->num_partitions < 0 || d->total_context < 0 || d->reuse_prefix_blocks < 0 ||
        d->window < 0 || d->sink_tokens < 0) {
        set_error("bad sizes: max_blocks_per_seq=%d num_blocks=%d max_context=%d",
                  d->max_blocks_per_seq, d->num_blocks, d->max_context);
        return PDA_EINVAL;
    }
    const bool eight = d->kv_dtype == PDA_FP8_E4M3 || d->kv_dtype == PDA_INT8;
    const bool wide = d->kv_dtype == PDA_F32 || d->kv_dtype == PDA_BF16;
    const bool int4 = d->kv_dtype == PDA_INT4;
    const bool kv_ok = kind == kQuant    ? eight
                       : kind == kPlain  ? wide
                       : kind == kPrefix ? (eight || d->kv_dtype == PDA_BF16)
                       : kind == kInt4   ? int4
                                         : (eight || wide || int4);
    if (!kv_ok) {
        set_error("kv_dtype %d not valid for this call", d->kv_dtype);
        return PDA_EINVAL;
    }
    if (d->prefix_blocks < 0 || d->prefix_blocks > d->max_blocks_per_seq ||
        d->prefix_blocks > kMaxPrefixBlocks) {
        set_error("prefix_blocks=%d outside [0, min(max_blocks_per_seq, %d)]", d->prefix_blocks,
                  kMaxPrefixBlocks);
        return PDA_EINVAL;
    }
    if (kind == kPrefix && d->prefix_blocks == 0) {
        set_error("shared-prefix call with prefix_blocks == 0");
        return PDA_EINVAL;
    }
    if (int4 && (d->window != 0 || d->prefix_blocks != 0)) {
        set_error("a 4-bit cache takes no window and no shared prefix");
        return PDA_EINVAL;
    }
    if ((kind == kPlain || kind == kQuant) && d->prefix_blocks != 0) {
        set_error("prefix_blocks=%d is for the *_prefix calls only", d->prefix_blocks);
        return PDA_EINVAL;
    }
    if (d->prefix_blocks > 0 && (d->window != 0 || d->kv_dtype == PDA_F32)) {
        set_error("a shared prefix needs window == 0 and a BF16 / FP8_E4M3 / INT8 cache");
        return PDA_EINVAL;
    }
    if ((d->q_dtype != PDA_F32 && d->q_dtype != PDA_BF16) ||
        (d->out_dtype != PDA_F32 && d->out_dtype != PDA_BF16)) {
        set_error("q_dtype / out_dtype must be F32 or BF16");
        return PDA_EINVAL;
    }
    // The stream kernel indexes its block axis (n_kv segments per row, each
    // up to max_blocks_per_seq blocks, plus a 4-bit cache's pad block and the
    // split units charged per segment) in 32 bits.
    if (d->kv_dtype != PDA_F32 &&
        (d->B > kMaxStreamBatch ||
         (int64_t)d->B * d->n_kv * ((int64_t)d->max_blocks_per_seq + 1 + kMaxSegCost) >=
             ((int64_t)1 << 31) ||
         (int64_t)d->B * d->n_kv >= ((int64_t)1 << 24))) {
        set_error("batch too large for one call: B <= %d and "
                  "B * n_kv * (max_blocks_per_seq + %d) < 2^31",
                  kMaxStreamBatch, 1 + kMaxSegCost);
        return PDA_EINVAL;
    }
    if ((int64_t)d->B * d->max_blocks_per_seq > INT32_MAX ||
        (int64_t)d->num_blocks * d->n_kv > INT32_MAX ||
        (int64_t)d->num_blocks * d->n_kv * kBlockSize * d->d_h * 4 > ((int64_t)1 << 46)) {
        set_error("sizes overflow the supported range");
        return PDA_EINVAL;
    }
    return PDA_OK;
}

// PDA_DEBUG: validate lengths and table entries on the host before launching,
// by the rule the kernels follow: a row is invalid if its length is outside
// [0, max_blocks * bs] or a block it looks up is unmapped (outside
// [0, num_blocks)). Looked up are, with a sliding window, only the sink
// blocks and the window's blocks; with a shared prefix of pl blocks, the
// prefix table's first pl entries instead of the row's own (and pl must be
// below the row's block count); with a 4-bit cache, the n / 16 encoded
// blocks (the open block is in the residual buffer).
int32_t debug_check(const pda_attn_desc* d, const int32_t* block_table,
                    const int32_t* context_lens, const int32_t* prefix_table,
                    const int32_t* prefix_lens, bool int4, hipStream_t s) {
    const bool prefix = prefix_table != nullptr;
    std::vector<int32_t> lens((size_t)d->B), table((size_t)d->B * d->max_blocks_per_seq);
    std::vector<int32_t> plens(prefix ? (size_t)d->B : 0), ptable(prefix ? (size_t)d->prefix_blocks : 0);
    hipError_t e = hipMemcpyAsync(lens.data(), context_lens, lens.size() * 4,
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(table.data(), block_table, table.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && prefix)
        e = hipMemcpyAsync(plens.data(), prefix_lens, plens.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && prefix)
        e = hipMemcpyAsync(ptable.data(), prefix_table, ptable.size() * 4, hipMemcpyDeviceToHost,
                           s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail("PDA_DEBUG copy", e);
    const int32_t sinks = d->window > 0 ? d->sink_tokens : 0;
    for (int32_t b = 0; b < d->B; ++b) {
        const int32_t n = lens[(size_t)b];
        if (n < 0 || (int64_t)n > (int64_t)d->max_blocks_per_seq * kBlockSize) {
            set_error("row %d: context length %d outside [0, %lld]", b, n,
                      (long long)d->max_blocks_per_seq * kBlockSize);
            return PDA_EINVAL;
        }
        const int32_t nblk = (n + kBlockSize - 1) / kBlockSize;
        int32_t pl = 0;
        if (prefix && n > 0) {
            pl = plens[(size_t)b];
            if (pl < 0 || pl > d->prefix_blocks || pl >= nblk) {
                set_error("row %d: shared-prefix length %d outside [0, min(%d, %d)]", b, pl,
                          d->prefix_blocks, nblk - 1);
                return PDA_EINVAL;
            }
            for (int32_t i = 0; i < pl; ++i) {
                const int32_t pb = ptable[(size_t)i];
                if (pb < 0 || pb >= d->num_blocks) {
                    set_error("row %d: shared-prefix block %d is unmapped (entry %d)", b, i, pb);
                    return PDA_EINVAL;
                }
            }
        }
        // attended blocks: all, or the sink blocks and those from the window's start
        int32_t sb = nblk, wstart = nblk;
        if (d->window > 0 && n > sinks + d->window) {
            sb = (sinks + kBlockSize - 1) / kBlockSize;
            wstart = std::max((n - d->window) / kBlockSize, sb);
        }
        const int32_t last = int4 ? n / kBlockSize : nblk;
        for (int32_t i = pl; i < last; ++i) {
            if (i >= sb && i < wstart) continue;
            const int32_t pb = table[(size_t)b * d->max_blocks_per_seq + i];
            if (pb < 0 || pb >= d->num_blocks) {
                set_error("row %d: logical block %d is unmapped (entry %d)", b, i, pb);
                return PDA_EINVAL;
            }
        }
    }
    return PDA_OK;
}

int32_t run_attn(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                 const float* v_scale, const int32_t* block_table, const int32_t* context_lens,
                 float scale, void* out, const pda_attn_desc* d, void* workspace,
                 size_t ws_bytes, void* stream, CallKind kind, const void* k_new = nullptr,
                 const void* v_new = nullptr, bool fused = false,
                 const int32_t* prefix_table = nullptr, const int32_t* prefix_lens = nullptr,
                 const void* k_res = nullptr, const void* v_res = nullptr) {
    int32_t rc = check_attn_desc(d, kind);
    if (rc != PDA_OK) return rc;
    const bool quant = d->kv_dtype == PDA_FP8_E4M3 || d->kv_dtype == PDA_INT8 ||
                       d->kv_dtype == PDA_INT4;
    if (fused) {
        const bool ok = quant ? (d->new_dtype == PDA_F32 || d->new_dtype == PDA_BF16)
                              : d->new_dtype == d->kv_dtype;
        if (!ok) {
            set_error("new_dtype %d does not fit the cache dtype %d", d->new_dtype, d->kv_dtype);
            return PDA_EINVAL;
        }
    }
    if (d->B == 0) return PDA_OK;
    if (fused && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))) {
        set_error("k_new / v_new must be 16-byte aligned device pointers");
        return PDA_EINVAL;
    }
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out ||
        (quant && (!k_scale || !v_scale)) ||
        (kind == kPrefix && (!prefix_table || !prefix_lens)) ||
        (kind == kInt4 && (!k_res || !v_res))) {
        set_error("NULL device pointer");
        return PDA_EINVAL;
    }
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) {
        set_error("q, caches and out must be 16-byte aligned");
        return PDA_EINVAL;
    }
    if (!std::isfinite(scale)) {
        set_error("scale is not finite");
        return PDA_EINVAL;
    }
    const Plan plan = make_plan(*d);
    const WsLayout ws = ws_layout(*d, plan);
    if (ws.bytes > 0 && (!workspace || ws_bytes < ws.bytes || !aligned16(workspace))) {
        set_error("workspace of %zu bytes needed (got %zu)", ws.bytes, ws_bytes);
        return PDA_EWORKSPACE;
    }
    hipStream_t s = (hipStream_t)stream;
    if (debug_mode()) {
        rc = debug_check(d, block_table, context_lens, kind == kPrefix ? prefix_table : nullptr,
                         prefix_lens, kind == kInt4, s);
        if (rc != PDA_OK) return rc;
    }
    AttnArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.out = out;
    a.part_o = ws.bytes ? (float*)((char*)workspace + ws.part_o_off) : nullptr;
    a.part_ml = ws.bytes ? (float*)((char*)workspace + ws.part_ml_off) : nullptr;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.B = d->B;
    a.n_q = d->n_q;
    a.n_kv = d->n_kv;
    a.g = d->n_q / d->n_kv;
    a.d_h = d->d_h;
    a.max_blocks = d->max_blocks_per_seq;
    a.num_blocks = d->num_blocks;
    a.kv_dtype = d->kv_dtype;
    a.q_dtype = d->q_dtype;
    a.out_dtype = d->out_dtype;
    a.seg_info = ws.bytes ? (int2*)((char*)workspace + ws.seg_info_off) : nullptr;
    a.P = plan.P;
    a.bpp = plan.bpp;
    a.nw = plan.nw;
    a.split = plan.split;
    a.reuse_blocks = d->reuse_prefix_blocks;
    a.window = d->window;
    a.sinks = d->window > 0 ? d->sink_tokens : 0;
    a.k_new = fused ? k_new : nullptr;
    a.v_new = fused ? v_new : nullptr;
    a.new_dtype = d->new_dtype;
    const bool prefix = kind == kPrefix;
    // Split units charged per (sequence, KV head) segment for its fixed costs
    // (a query load, a partial write, a fused append). Measured on MI355X:
    // with a shared prefix many rows keep only a block or two of their own,
    // and a wave crossing dozens of such segments set the kernel's time until
    // each segment start was charged as 4 blocks; with whole rows the
    // segments are long and equal block counts per wave are best.
    a.seg_cost = std::min(std::max(env_int("PDA_SEGMENT_COST", prefix ? 4 : 0), 0), kMaxSegCost);
    a.prefix_table = prefix ? prefix_table : nullptr;
    a.prefix_lens = prefix ? prefix_lens : nullptr;
    a.prefix_blocks = prefix ? d->prefix_blocks : 0;
    const bool int4 = kind == kInt4;
    a.pre_o = prefix ? (float*)((char*)workspace + ws.pre_o_off) : nullptr;
    a.pre_ml = prefix ? (float*)((char*)workspace + ws.pre_ml_off) : nullptr;
    a.k_res = int4 ? k_res : nullptr;
    a.v_res = int4 ? v_res : nullptr;
    a.extra_pieces = int4 ? 1 : 0;
    hipError_t e;
    if (prefix) {
        // the shared blocks first: they are never the block a fused step writes
        e = launch_attn_prefix(a, s);
        if (e != hipSuccess) return hip_fail("prefix attention launch", e);
    }
    if (plan.stream) {
        e = launch_attn_mfma(a, s);
        if (e != hipSuccess) return hip_fail("attention launch", e);
        if (plan.split) {
            e = launch_merge_stream(a, s);
            if (e != hipSuccess) return hip_fail("merge launch", e);
        }
        return PDA_OK;
    }
    e = launch_attn_f32(a, s);
    if (e != hipSuccess) return hip_fail("attention launch", e);
    if (plan.P > 1) {
        e = launch_merge_for_attn(a, s);
        if (e != hipSuccess) return hip_fail("merge launch", e);
    }
    return PDA_OK;
}

int32_t check_kv_desc(const pda_kv_desc* d, bool quant) {
    if (!d || d->n_kv <= 0 || (d->d_h != 64 && d->d_h != 128) || d->block_size != kBlockSize ||
        d->num_blocks <= 0) {
        set_error("bad KV descriptor");
        return PDA_EINVAL;
    }
    if (quant) {
        if ((d->cache_dtype != PDA_FP8_E4M3 && d->cache_dtype != PDA_INT8) ||
            (d->src_dtype != PDA_F32 && d->src_dtype != PDA_BF16)) {
            set_error("quantized append: cache FP8_E4M3/INT8, source F32/BF16");
            return PDA_EINVAL;
        }
    } else if ((d->cache_dtype != PDA_F32 && d->cache_dtype != PDA_BF16) ||
               d->src_dtype != d->cache_dtype) {
        set_error("append: cache F32/BF16 and source of the same dtype");
        return PDA_EINVAL;
    }
    return PDA_OK;
}

}  // namespace

extern "C" {

const char* pda_version(void) { return "pda 0.1.0 (gfx950)"; }

const char* pda_last_error(void) { return pda::g_err; }

int32_t pda_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache, const pda_kv_desc* d,
                      void* stream) {
    int32_t rc = check_kv_desc(d, false);
    if (rc != PDA_OK) return rc;
    if (num_tokens < 0) {
        set_error("num_tokens < 0");
        return PDA_EINVAL;
    }
    if (num_tokens == 0) return PDA_OK;
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) {
        set_error("NULL device pointer");
        return PDA_EINVAL;
    }
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)) {
        set_error("K/V buffers must be 16-byte aligned");
        return PDA_EINVAL;
    }
    AppendArgs a{k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, nullptr, nullptr,
                 d->n_kv, d->d_h, d->block_size, d->num_blocks, d->cache_dtype, d->src_dtype};
    hipError_t e = launch_append(a, (hipStream_t)stream);
    return e == hipSuccess ? PDA_OK : hip_fail("append launch", e);
}

int32_t pda_kv_append_quant(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                            int32_t num_tokens, void* k_cache, void* v_cache,
                            const float* k_scale, const float* v_scale, const pda_kv_desc* d,
                            void* stream) {
    int32_t rc = check_kv_desc(d, true);
    if (rc != PDA_OK) return rc;
    if (num_tokens < 0) {
        set_error("num_tokens < 0");
        return PDA_EINVAL;
    }
    if (num_tokens == 0) return PDA_OK;
    if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale) {
        set_error("NULL device pointer");
        return PDA_EINVAL;
    }
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)) {
        set_error("K/V buffers must be 16-byte aligned");
        return PDA_EINVAL;
    }
    AppendArgs a{k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, k_scale, v_scale,
                 d->n_kv, d->d_h, d->block_size, d->num_blocks, d->cache_dtype, d->src_dtype};
    hipError_t e = launch_append_quant(a, (hipStream_t)stream);
    return e == hipSuccess ? PDA_OK : hip_fail("quantized append launch", e);
}

int32_t pda_attn_workspace_size(const pda_attn_desc* d, size_t* bytes) {
    if (!bytes) {
        set_error("bytes is NULL");
        return PDA_EINVAL;
    }
    int32_t rc = check_attn_desc(d, kQuery);
    if (rc != PDA_OK) return rc;
    *bytes = ws_layout(*d, make_plan(*d)).bytes;
    return PDA_OK;
}

int32_t pda_attn_plan(const pda_attn_desc* d, int32_t* num_partitions,
                      int32_t* blocks_per_partition) {
    if (!num_partitions || !blocks_per_partition) {
        set_error("NULL output pointer");
        return PDA_EINVAL;
    }
    int32_t rc = check_attn_desc(d, kQuery);
    if (rc != PDA_OK) return rc;
    const Plan p = make_plan(*d);
    *num_partitions = p.P;
    *blocks_per_partition = p.bpp;
    return PDA_OK;
}

int32_t pda_paged_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* context_lens, float scale,
                              void* out, const pda_attn_desc* d, void* workspace,
                              size_t ws_bytes, void* stream) {
    return run_attn(q, k_cache, v_cache, nullptr, nullptr, block_table, context_lens, scale, out,
                    d, workspace, ws_bytes, stream, kPlain);
}

int32_t pda_paged_decode_attn_quant(const void* q, const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* block_table, const int32_t* context_lens,
                                    float scale, void* out, const pda_attn_desc* d,
                                    void* workspace, size_t ws_bytes, void* stream) {
    return run_attn(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, scale, out,
                    d, workspace, ws_bytes, stream, kQuant);
}

int32_t pda_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                        void* v_cache, const int32_t* block_table, const int32_t* context_lens,
                        float scale, void* out, const pda_attn_desc* d, void* workspace,
                        size_t ws_bytes, void* stream) {
    return run_attn(q, k_cache, v_cache, nullptr, nullptr, block_table, context_lens, scale, out,
                    d, workspace, ws_bytes, stream, kPlain, k_new, v_new, true);
}

int32_t pda_decode_step_quant(const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, const float* k_scale,
                              const float* v_scale, const int32_t* block_table,
                              const int32_t* context_lens, float scale, void* out,
                              const pda_attn_desc* d, void* workspace, size_t ws_bytes,
                              void* stream) {
    return run_attn(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, scale, out,
                    d, workspace, ws_bytes, stream, kQuant, k_new, v_new, true);
}

int32_t pda_paged_decode_attn_prefix(const void* q, const void* k_cache, const void* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_table, const int32_t* context_lens,
                                     const int32_t* prefix_table, const int32_t* prefix_lens,
                                     float scale, void* out, const pda_attn_desc* d,
                                     void* workspace, size_t ws_bytes, void* stream) {
    return run_attn(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, scale, out,
                    d, workspace, ws_bytes, stream, kPrefix, nullptr, nullptr, false,
                    prefix_table, prefix_lens);
}

int32_t pda_decode_step_prefix(const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, const float* k_scale,
                               const float* v_scale, const int32_t* block_table,
                               const int32_t* context_lens, const int32_t* prefix_table,
                               const int32_t* prefix_lens, float scale, void* out,
                               const pda_attn_desc* d, void* workspace, size_t ws_bytes,
                               void* stream) {
    return run_attn(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, scale, out,
                    d, workspace, ws_bytes, stream, kPrefix, k_new, v_new, true, prefix_table,
                    prefix_lens);
}

int32_t pda_paged_decode_attn_int4(const void* q, const void* k_q, const void* v_q,
                                   const float* k_scale, const float* v_scale,
                                   const void* k_res, const void* v_res,
                                   const int32_t* block_table, const int32_t* context_lens,
                                   float scale, void* out, const pda_attn_desc* d,
                                   void* workspace, size_t ws_bytes, void* stream) {
    if ((k_res && !aligned16(k_res)) || (v_res && !aligned16(v_res)) ||
        (k_scale && !aligned16(k_scale)) || (v_scale && !aligned16(v_scale))) {
        set_error("k_res, v_res, k_scale and v_scale must be 16-byte aligned");
        return PDA_EINVAL;
    }
    return run_attn(q, k_q, v_q, k_scale, v_scale, block_table, context_lens, scale, out, d,
                    workspace, ws_bytes, stream, kInt4, nullptr, nullptr, false, nullptr, nullptr,
                    k_res, v_res);
}

int32_t pda_decode_step_int4(const void* q, const void* k_new, const void* v_new, void* k_q,
                             void* v_q, const float* k_scale, float* v_scale, void* k_res,
                             void* v_res, const int32_t* block_table,
                             const int32_t* context_lens, float scale, void* out,
                             const pda_attn_desc* d, void* workspace, size_t ws_bytes,
                             void* stream) {
    if (d && d->new_dtype != PDA_BF16) {
        set_error("a fused 4-bit step takes bf16 k_new / v_new (new_dtype %d)", d->new_dtype);
        return PDA_EINVAL;
    }
    if ((k_res && !aligned16(k_res)) || (v_res && !aligned16(v_res)) ||
        (k_scale && !aligned16(k_scale)) || (v_scale && !aligned16(v_scale))) {
        set_error("k_res, v_res, k_scale and v_scale must be 16-byte aligned");
        return PDA_EINVAL;
    }
    return run_attn(q, k_q, v_q, k_scale, v_scale, block_table, context_lens, scale, out, d,
                    workspace, ws_bytes, stream, kInt4, k_new, v_new, true, nullptr, nullptr,
                    k_res, v_res);
}

int32_t pda_kv_append_int4(const void* k_new, const void* v_new, const int32_t* block_table,
                           const int32_t* context_lens, void* k_q, void* v_q,
                           const float* k_scale, float* v_scale, void* k_res, void* v_res,
                           const pda_attn_desc* d, void* stream) {
    int32_t rc = check_attn_desc(d, kInt4);
    if (rc != PDA_OK) return rc;
    if (d->B == 0) return PDA_OK;
    if (!k_new || !v_new || !block_table || !context_lens || !k_q || !v_q || !k_scale ||
        !v_scale || !k_res || !v_res) {
        set_error("NULL device pointer");
        return PDA_EINVAL;
    }
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_q) || !aligned16(v_q) ||
        !aligned16(k_res) || !aligned16(v_res) || !aligned16(k_scale) || !aligned16(v_scale)) {
        set_error("int4 append buffers must be 16-byte aligned");
        return PDA_EINVAL;
    }
    hipError_t e = launch_append_int4(k_new, v_new, block_table, context_lens, k_q, v_q, k_scale,
                                      v_scale, k_res, v_res, d->B, d->n_kv, d->d_h,
                                      d->max_blocks_per_seq, d->num_blocks, (hipStream_t)stream);
    return e == hipSuccess ? PDA_OK : hip_fail("int4 append launch", e);
}

int32_t pda_lse_merge(const float* part_o, const float* part_ml, int32_t rows, int32_t P,
                      int32_t d_h, float* out, void* stream) {
    if (rows < 0 || P < 1 || P > kMaxPartitions || (d_h != 64 && d_h != 128)) {
        set_error("pda_lse_merge: rows >= 0, 1 <= P <= %d, d_h 64 or 128", kMaxPartitions);
        return PDA_EINVAL;
    }
    if (rows == 0) return PDA_OK;
    if (!part_o || !part_ml || !out) {
        set_error("NULL device pointer");
        return PDA_EINVAL;
    }
    if (!aligned16(part_o) || !aligned16(out) || ((uintptr_t)part_ml & 7u) != 0) {
        set_error("part_o and out must be 16-byte aligned, part_ml 8-byte aligned");
        return PDA_EINVAL;
    }
    hipError_t e = launch_lse_merge(part_o, part_ml, rows, P, d_h, out, (hipStream_t)stream);
    return e == hipSuccess ? PDA_OK : hip_fail("merge launch", e);
}

int32_t pda_hbm_read_probe(const void* buf, size_t bytes, const int64_t* tile_offsets,
                           int64_t n_tiles, int32_t tile_bytes, int32_t waves, uint32_t* sink,
                           void* stream) {
    if (!buf || !sink || !aligned16(buf) || waves < 4 || waves > 65536 || waves % 4 != 0) {
        set_error("read probe: buf and sink non-NULL, buf 16-byte aligned, waves a multiple "
                  "of 4 in [4, 65536]");
        return PDA_EINVAL;
    }
    if (tile_offsets == nullptr) {
        if (bytes / 4096 < (size_t)waves) {
            set_error("read probe: %zu bytes is less than one 4 KiB step per wave", bytes);
            return PDA_EINVAL;
        }
    } else if (n_tiles < 0 || (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096 &&
                               tile_bytes != 8192) || (size_t)tile_bytes > bytes) {
        set_error("read probe: n_tiles >= 0 and tile_bytes 1024, 2048, 4096 or 8192");
        return PDA_EINVAL;
    }
    hipError_t e = launch_read_probe(buf, bytes, tile_offsets, n_tiles, tile_bytes, waves, sink,
                                     (hipStream_t)stream);
    return e == hipSuccess ? PDA_OK : hip_fail("read probe launch", e);
}

}  // extern "C"
