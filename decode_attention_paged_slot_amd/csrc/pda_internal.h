// pda_internal.h -- host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda.h"

namespace pda {

void set_error(const char* fmt, ...);

// Split plan.
//  fp32 caches (partition plan): P partitions of `bpp` logical blocks per
//    sequence, grid (P, n_q, B).
//  16-bit and 8-bit caches (stream plan): split = 1 cuts the flattened
//    (sequence, KV head, block) axis into `nw` equal wave ranges; split = 0
//    gives one wave per (sequence, KV head). P reports nw when split, else 1;
//    bpp the expected blocks per range.
struct Plan {
    int32_t P;
    int32_t bpp;
    int32_t nw;
    int32_t split;
    int32_t stream;
};
Plan make_plan(const pda_attn_desc& d);

// Workspace layout for a plan.
struct WsLayout {
    size_t part_o_off, part_ml_off, seg_info_off, pre_o_off, pre_ml_off, bytes;
};
WsLayout ws_layout(const pda_attn_desc& d, const Plan& p);

struct AppendArgs {
    const void* k_new;
    const void* v_new;
    const int64_t* slots;
    int32_t T;
    void* k_cache;
    void* v_cache;
    const float* k_scale;
    const float* v_scale;
    int32_t n_kv, d_h, bs, num_blocks, cache_dtype, src_dtype;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_quant(const AppendArgs& a, hipStream_t s);

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_table;
    const int32_t* context_lens;
    void* out;
    float* part_o;   // partition plan: [B][n_q][P][d_h]; stream plan: [S + nw][g][d_h]
    float* part_ml;  // partition plan: [B][n_q][P][2];   stream plan: [S + nw][g][2]
    int2* seg_info;  // stream plan: [S] (first wave, last wave) of each segment
    float scale_log2;  // softmax scale * log2(e)
    int32_t B, n_q, n_kv, g, d_h, max_blocks, num_blocks;
    int32_t kv_dtype, q_dtype, out_dtype;
    int32_t P, bpp;
    int32_t nw, split;
    int32_t seg_cost;       // stream split: extra units per non-empty segment
    int32_t reuse_blocks;   // leading logical blocks read with cache-retaining loads
    int32_t window, sinks;  // sliding window (0 = all positions) and its sink tokens
    // fused decode step: the new rows [B][n_kv][d_h] of new_dtype, written into
    // position n - 1 of each row (nullptr: attention only)
    const void* k_new;
    const void* v_new;
    int32_t new_dtype;
    // shared prefix (nullptr / 0: none): logical blocks i < prefix_lens[b] of
    // row b are prefix_table[i]; the prefix pass writes one partial per
    // (chunk of kPrefixChunk prefix blocks, output row) to pre_o / pre_ml
    const int32_t* prefix_table;
    const int32_t* prefix_lens;
    int32_t prefix_blocks;
    float* pre_o;    // [chunks][B * n_q][d_h]
    float* pre_ml;   // [chunks][B * n_q][2]
    // 4-bit cache (kv_dtype DT_INT4): k_scale is [n_kv][d_h] (per channel),
    // v_scale [num_blocks][n_kv][16] (per token); each row's open block is in
    // k_res / v_res [B][n_kv][16][d_h] bf16 (extra_pieces = 1): the merge
    // attends it as one more piece of every row with n % 16 != 0
    const void* k_res;
    const void* v_res;
    int32_t extra_pieces;
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_prefix(const AttnArgs& a, hipStream_t s);
hipError_t launch_append_int4(const void* k_new, const void* v_new, const int32_t* block_table,
                              const int32_t* context_lens, void* k_q, void* v_q,
                              const float* k_scale, float* v_scale, void* k_res, void* v_res,
                              int32_t B, int32_t n_kv, int32_t d_h, int32_t max_blocks,
                              int32_t num_blocks, hipStream_t s);
hipError_t launch_merge_for_attn(const AttnArgs& a, hipStream_t s);
hipError_t launch_merge_stream(const AttnArgs& a, hipStream_t s);
size_t attn_mfma_dyn_lds(int32_t B, bool prefix);
hipError_t launch_read_probe(const void* buf, size_t bytes, const int64_t* tile_offsets,
                             int64_t n_tiles, int32_t tile_bytes, int32_t waves,
                             uint32_t* sink, hipStream_t s);
hipError_t launch_lse_merge(const float* part_o, const float* part_ml, int32_t rows, int32_t P,
                            int32_t d_h, float* out, hipStream_t s);

constexpr int kBlockSize = 16;
constexpr int kMaxPartitions = 2048;
constexpr int kMaxStreamBatch = 4096;      // sequences per call on the stream plan (LDS prefix)
constexpr int kMaxStreamWaves = 8192;      // wave ranges on the stream plan (merge LDS)
constexpr int kMaxSegCost = 64;            // split units charged per segment, at most
constexpr int kAttnThreads = 256;
constexpr int kPrefixChunk = 16;           // shared-prefix blocks per prefix-pass workgroup
constexpr int kMaxPrefixBlocks = 32768;    // shared-prefix blocks per call (merge LDS)

}  // namespace pda
