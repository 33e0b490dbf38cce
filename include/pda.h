/*
 * pda.h -- C ABI of the paged decode-attention library for AMD MI355X (gfx950).
 *
 * One decode step of one attention layer: the step's new keys/values are
 * appended into their mapped cache slots, then every sequence's single new
 * query attends over its whole cached history through a block table.
 *
 * The method, in the pages' terms:
 *  - The KV cache keeps each layer's keys and values in HBM; each processed
 *    token appends one K and one V row (the append path), and every decode
 *    step rereads the prior rows (the read path)  ["9 Decode and KV Cache",
 *    section 9.4].
 *  - Paged allocation: fixed-size blocks, a per-request block table maps
 *    logical blocks to physical blocks; a logical position resolves to
 *    (table[pos / bs], pos % bs) before the kernel reads KV memory; the
 *    attention arithmetic itself is unchanged by paging  [section 9.5,
 *    including its block-lookup example].
 *  - Grouped-query attention: g = n_q / n_kv query heads address one stored
 *    KV head  [GQA teaser on the kv-cache tag page; SoK paper section 1.1].
 *  - A quantized cache stores fewer bits per element plus scale metadata and
 *    is reconstructed when attention consumes it  [KV-cache quantization
 *    teasers on the kv-cache tag page; SoK paper sections 2.3 and 5.2].
 *  - Decode attention is memory bound: 2 g / w_kv FLOP per KV byte  [SoK
 *    paper section 1.1; "9 Decode and KV Cache", section 9.3].
 *
 * Conventions for every call:
 *  - All functions return a pda_status and never throw or abort.
 *  - "device" pointers are HIP device memory of the current device; "host"
 *    pointers are ordinary CPU memory. The caller allocates and owns every
 *    buffer, including the attention workspace; the library allocates no
 *    device memory on any path.
 *  - Device work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) with no implicit synchronisation. Input buffers are read-only.
 *  - Dtype codes (pda_dtype): PDA_F32 IEEE binary32; PDA_BF16 bfloat16;
 *    PDA_FP8_E4M3 OCP 8-bit E4M3 (bias 7, max +-448, S.1111.111 = NaN, no
 *    infinities); PDA_INT8 two's-complement, symmetric (value = scale * code).
 *  - Supported: d_h in {64, 128}; block_size == 16 (the block size the SoK
 *    paper's paging domain names, section 2.5); 1 <= n_q / n_kv <= 16.
 *  - The kernels apply no positional transform: cached keys already carry
 *    their rotation (RoPE teaser on the kv-cache tag page).
 *  - On PDA_EHIP, pda_last_error() names the HIP error.
 */
#ifndef PDA_H
#define PDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pda_status {
    PDA_OK = 0,
    PDA_EINVAL = 1,      /* null pointer, bad size, unsupported shape/dtype, non-finite scale */
    PDA_ENOSPC = 2,      /* block pool exhausted: the preemption signal (section 9.5) */
    PDA_EWORKSPACE = 3,  /* attention workspace smaller than pda_attn_workspace_size() */
    PDA_EHIP = 4         /* a HIP call failed; see pda_last_error() */
} pda_status;

typedef enum pda_dtype {
    PDA_F32 = 0,
    PDA_BF16 = 1,
    PDA_FP8_E4M3 = 2,
    PDA_INT8 = 3,
    PDA_INT4 = 4      /* 4-bit cache with a bf16 residual window (pda_*_int4 calls) */
} pda_dtype;

/* ------------------------------------------------------------------ misc */

/* Library version string (static storage). */
const char* pda_version(void);

/* Text of the last error recorded on the calling thread ("" if none). */
const char* pda_last_error(void);

/* ------------------------------------------------------- host block pool
 * Fixed-size blocks allocated on demand from a free list, with reference
 * counts so several tables may share a block (prefix sharing / copy on
 * write)  [section 9.5; SoK paper sections 2.5-2.6]. Host memory only; not
 * thread-safe (the caller serialises calls on one pool).
 *
 * The free list is FIFO: allocation takes ids from its front, and a block
 * whose last reference is released goes to its back. Its initial order is the
 * caller's `free_order` (a permutation of 0..num_blocks-1; NULL = ascending),
 * so random physical placement is an input, reproducible from one seed.
 */
typedef struct pda_pool pda_pool;

/* Create a pool of num_blocks (>= 1) blocks. free_order: host [num_blocks]
 * permutation or NULL. *out receives the pool (owned by the caller; release
 * with pda_pool_destroy). EINVAL if free_order is not a permutation. */
int32_t pda_pool_create(int32_t num_blocks, const int32_t* free_order, pda_pool** out);

/* Destroy a pool (NULL is a no-op). */
int32_t pda_pool_destroy(pda_pool* pool);

/* Allocate n blocks from the front of the free list, refcount 1 each, ids in
 * allocation order to host ids_out[n]. All-or-nothing: if fewer than n are
 * free, returns PDA_ENOSPC and changes nothing. */
int32_t pda_pool_alloc(pda_pool* pool, int32_t n, int32_t* ids_out);

/* Add one reference to each listed block (host ids[n]); every id must be
 * allocated, else EINVAL with no change. */
int32_t pda_pool_share(pda_pool* pool, int32_t n, const int32_t* ids);

/* Drop one reference from each listed block; blocks reaching zero return to
 * the back of the free list in the order listed. EINVAL (no change) if any id
 * would be released more often than it is referenced. */
int32_t pda_pool_free(pda_pool* pool, int32_t n, const int32_t* ids);

/* Number of free blocks. */
int32_t pda_pool_num_free(const pda_pool* pool, int32_t* out);

/* Reference count of block id (0 = free). */
int32_t pda_pool_refcount(const pda_pool* pool, int32_t id, int32_t* out);

/* Build block tables and the slot of each row's newest token.
 *   context_lens  host [B]: tokens of row b, INCLUDING the token appended
 *                 this step (the current input token is attended,
 *                 section 9.1); 0 = empty row.
 *   shared_ids    host [n_shared] already-allocated blocks holding a common
 *                 prefix; row b reuses the first min(n_shared, blocks_b - 1)
 *                 of them (one more reference each). The block receiving the
 *                 row's newest token is always private (copy on write).
 *   block_table_out host [B][max_blocks]: row b's physical blocks for logical
 *                 blocks 0..blocks_b-1, then -1.
 *   slot_mapping_out host [B]: table[b][(n-1)/bs] * bs + (n-1) % bs, the flat
 *                 cache row of the newest token (worked example "PagedAttention
 *                 block lookup", section 9.5); -1 for an empty row.
 * Fresh blocks come from the pool in row order. All-or-nothing: ENOSPC if the
 * pool cannot supply every fresh block, EINVAL if a row needs more than
 * max_blocks blocks or a shared id is not allocated; nothing changes then. */
int32_t pda_build_block_table(pda_pool* pool, int32_t B, const int32_t* context_lens,
                              int32_t block_size, int32_t n_shared, const int32_t* shared_ids,
                              int32_t max_blocks, int32_t* block_table_out,
                              int64_t* slot_mapping_out);

/* ---------------------------------------------------------- KV append
 * Cache layout (both K and V, row-major): [num_blocks][n_kv][block_size][d_h]
 * elements of cache_dtype; one (block, head) tile is one contiguous run of
 * block_size * d_h elements. Slot s addresses row (s / bs, :, s % bs, :).
 */
typedef struct pda_kv_desc {
    int32_t n_kv;          /* KV heads */
    int32_t d_h;           /* head dimension (64 or 128) */
    int32_t block_size;    /* tokens per block (16) */
    int32_t num_blocks;    /* physical blocks in the cache */
    int32_t cache_dtype;   /* pda_dtype of the cache */
    int32_t src_dtype;     /* pda_dtype of k_new / v_new (PDA_F32 or PDA_BF16) */
} pda_kv_desc;

/* Append path [section 9.4]: for t < num_tokens and every KV head h,
 *   k_cache[slot/bs][h][slot%bs][:] = k_new[t][h][:]   (bit copy; same for V)
 * with slot = slot_mapping[t]. A negative slot is a padding token and writes
 * nothing; a slot >= num_blocks * block_size is skipped as well.
 *   k_new, v_new   device [num_tokens][n_kv][d_h], src_dtype == cache_dtype
 *                  (PDA_F32 or PDA_BF16)
 *   slot_mapping   device [num_tokens] int64
 *   k_cache, v_cache device caches (layout above), written in place
 * num_tokens == 0 returns PDA_OK without launching. Duplicate slots in one
 * call are a caller error (the surviving row is unspecified). */
int32_t pda_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache, const pda_kv_desc* d,
                      void* stream);

/* Quantized append: the new rows are encoded with their destination block's
 * per-(block, KV head) scale and stored as 8-bit codes  [KV-cache
 * quantization teasers: entries are encoded with fewer bits and
 * reconstructed when attention consumes them].
 *   cache_dtype    PDA_FP8_E4M3 or PDA_INT8; src_dtype PDA_F32 or PDA_BF16
 *   k_scale, v_scale device [num_blocks][n_kv] fp32, owned and set by the
 *                  caller when it opens a block (must be positive and finite)
 * Per element: y = fp32(x) * fp32(1 / scale) (IEEE fp32 reciprocal, then one
 * fp32 multiply), code = round-to-nearest-even with saturation:
 *   fp8: nearest finite E4M3 value (|y| > 448 -> +-448; NaN -> 0x7F; the sign
 *        of y is kept, so -0 -> 0x80);
 *   int8: rint(y) clamped to [-127, 127]; NaN -> 0.
 * Slots as for pda_kv_append. */
int32_t pda_kv_append_quant(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                            int32_t num_tokens, void* k_cache, void* v_cache,
                            const float* k_scale, const float* v_scale, const pda_kv_desc* d,
                            void* stream);

/* ------------------------------------------------- paged decode attention */
typedef struct pda_attn_desc {
    int32_t B;                  /* sequences (rows of the batch) */
    int32_t n_q;                /* query heads */
    int32_t n_kv;               /* KV heads; n_q % n_kv == 0, g = n_q / n_kv in 1..16 */
    int32_t d_h;                /* head dimension (64 or 128) */
    int32_t block_size;         /* 16 */
    int32_t max_blocks_per_seq; /* columns of block_table */
    int32_t num_blocks;         /* physical blocks in the cache */
    int32_t kv_dtype;           /* pda_dtype of the caches */
    int32_t q_dtype;            /* PDA_F32 or PDA_BF16 */
    int32_t out_dtype;          /* PDA_F32 or PDA_BF16 (round to nearest even) */
    int32_t max_context;        /* host-side bound on context_lens, sizes the split */
    int32_t num_partitions;     /* split-KV partitions: 0 = choose, 1 = none, k = at most k */
    int64_t total_context;      /* optional sum of context_lens (0 = unknown); tunes the split */
    int32_t reuse_prefix_blocks; /* cache hint: the first reuse_prefix_blocks logical blocks
                                    of every row are read with cache-retaining loads (blocks
                                    shared by many rows, e.g. a common prompt prefix, are then
                                    served from L2 / Infinity Cache after their first read);
                                    all other blocks are streamed with non-temporal loads.
                                    0 = stream everything. Affects speed only, never results. */
    int32_t window;             /* sliding window: > 0 attends only to the last `window`
                                   positions of each row, plus its first sink_tokens
                                   positions; 0 = every position  ["9 Decode and KV Cache",
                                   section 9.7; sink and sliding-window teasers] */
    int32_t sink_tokens;        /* attention sinks kept with a window (ignored if window == 0) */
    int32_t new_dtype;          /* pda_decode_step*: pda_dtype of k_new / v_new (PDA_F32 or
                                   PDA_BF16; equal to kv_dtype for 16/32-bit caches) */
    int32_t prefix_blocks;      /* *_prefix calls: entries of prefix_table (the longest
                                   shared prefix, in blocks, <= max_blocks_per_seq); sizes
                                   the workspace. Must be 0 for every other call. */
} pda_attn_desc;

/* Workspace bytes the attention calls need for this descriptor (0 when the
 * call runs unsplit and without a shared prefix). The workspace holds the
 * split-KV partial results (normalised output, max, sum per piece) and the
 * split bookkeeping; its layout is internal to the library and nothing in
 * it needs clearing between calls. A call writes the workspace and then
 * reads it back in a later kernel on the same stream, so two calls that may
 * run at the same time (on different streams) need separate workspaces;
 * calls ordered on one stream can share one. Host-only. */
int32_t pda_attn_workspace_size(const pda_attn_desc* d, size_t* bytes);

/* The split chosen for this descriptor: *num_partitions = P (1 = unsplit) and
 * *blocks_per_partition = logical blocks per partition (each a contiguous
 * logical token range; row b uses ceil(ceil(n_b / bs) / bpp) of them).
 * Host-only. */
int32_t pda_attn_plan(const pda_attn_desc* d, int32_t* num_partitions,
                      int32_t* blocks_per_partition);

/* Paged decode attention  [sections 9.4-9.5; SoK paper section 1.1]: for
 * every row b and query head h, with j = h / g and n = context_lens[b],
 *   s_t   = scale * <q[b][h], K[pb(t)][j][t % bs]>,  pb(t) = block_table[b][t / bs]
 *   out[b][h] = sum_{t in A} softmax(s)_t * V[pb(t)][j][t % bs]
 * over the attended positions A = { t < n } (window == 0), or with a sliding
 * window A = { t < n : t < sink_tokens or t >= n - window } (section 9.7);
 * positions outside A are never looked up or read.
 * evaluated in fp32 with exact-product matrix-core accumulation; the cache is
 * read once per step and no score is written to memory (SoK appendices A.1,
 * C.4). Long contexts are split into partitions whose partial results are
 * merged by a log-sum-exp merge in the same call.
 *   q            device [B][n_q][d_h], q_dtype
 *   k_cache, v_cache device caches (layout of pda_kv_desc), kv_dtype F32/BF16
 *   block_table  device [B][max_blocks_per_seq] int32; entries past a row's
 *                ceil(n / bs) are never read
 *   context_lens device [B] int32 (includes the token appended this step)
 *   scale        softmax scale (finite), e.g. 1 / sqrt(d_h)
 *   out          device [B][n_q][d_h], out_dtype
 *   workspace    device, ws_bytes >= pda_attn_workspace_size(d) (NULL if 0)
 * Row semantics: n == 0 -> zero row. A logical block whose table entry is
 * outside [0, num_blocks), or n < 0, or n > max_blocks_per_seq * bs, is an
 * error (the worked example's failing lookup): that row's output is NaN.
 * Rows may share physical blocks (read-only aliasing). One call takes at
 * most 4096 sequences (16-bit, 8-bit and 4-bit caches) with
 * B * n_kv * (max_blocks_per_seq + 65) < 2^31 (EINVAL beyond). Errors: EINVAL,
 * EWORKSPACE, EHIP. With PDA_DEBUG=1 in the environment the host also copies
 * block_table / context_lens back (synchronising `stream`) and returns EINVAL
 * for any such row before launching. It checks the blocks the call looks up,
 * as the kernels do: blocks a sliding window skips are not looked up (nor,
 * in the _prefix calls, a row's own entries below its prefix length, nor, in
 * the _int4 calls, a row's open block).
 * Tuning overrides, read from the environment at each call and by
 * pda_attn_workspace_size, so keep them fixed between the two (defaults are
 * the measured best on MI355X; any value gives a correct result, only the
 * split, and with it the rounding order, changes):
 *   PDA_ATTN_WORKGROUPS      workgroups of the split (4 wave ranges each);
 *                            default one per compute unit of the current
 *                            device (256 on an MI355X) for 16-bit caches,
 *                            two per compute unit for 8-bit and 4-bit ones
 *   PDA_MIN_BLOCKS_PER_WAVE  fewest expected blocks per wave range before the
 *                            split shrinks the wave count (default 8)
 *   PDA_SEGMENT_COST         extra units charged per (sequence, KV head)
 *                            segment when ranges are cut (default 0; 4 for
 *                            the _prefix calls; at most 64) */
int32_t pda_paged_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* context_lens, float scale,
                              void* out, const pda_attn_desc* d, void* workspace,
                              size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as pda_paged_decode_attn, with the workspace taken from a fixed
 * device array of the library instead of the caller. Nothing is allocated:
 * no hipMalloc, hipFree or allocating library routine is called. The array
 * holds PDA_NOALLOC_SCRATCH_BYTES bytes on every device the library runs
 * on, kept until the process ends; its device address is looked up once per
 * device, on the first call with that device current. A descriptor whose
 * pda_attn_workspace_size exceeds the limit returns PDA_EWORKSPACE (use
 * pda_paged_decode_attn with a caller workspace then). The array needs no
 * clearing between calls. All calls on one device share its array, so two
 * such calls whose kernels may overlap (different streams of one device)
 * race and corrupt each other's results; order them on one stream.
 * Arguments, row semantics and other errors as for pda_paged_decode_attn
 * (f32 and bf16 caches). */
#define PDA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int32_t pda_paged_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* context_lens,
                                      float scale, void* out, const pda_attn_desc* d,
                                      void* stream);

/* Quantized-cache variant: kv_dtype PDA_FP8_E4M3 or PDA_INT8 and
 *   K = k_scale[pb][j] * dec(K_code),  V = v_scale[pb][j] * dec(V_code)
 * with k_scale, v_scale device [num_blocks][n_kv] fp32. The scales are folded
 * into the score and into the probability weights (no expanded copy of the
 * cache is ever written)  [SoK paper section 5.2]. Otherwise as above. */
int32_t pda_paged_decode_attn_quant(const void* q, const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* block_table, const int32_t* context_lens,
                                    float scale, void* out, const pda_attn_desc* d,
                                    void* workspace, size_t ws_bytes, void* stream);

/* One fused decode step: the append of each row's new token followed by
 * paged decode attention, in one launch  [section 9.4: append path and read
 * path of the same step]. For every row b with n = context_lens[b] > 0 and
 * every KV head j, position n - 1 of the row (slot
 * block_table[b][(n-1)/bs] * bs + (n-1) % bs, as the block-table builder
 * maps it) receives k_new[b][j][:] / v_new[b][j][:], and the attention of
 * row b then includes it. The result, in `out` and in the caches, is bit for
 * bit that of pda_kv_append (slot_mapping as above) followed by
 * pda_paged_decode_attn; rows with n == 0 or an invalid n append nothing.
 *   k_new, v_new  device [B][n_kv][d_h], d->new_dtype (== kv_dtype here)
 *   k_cache, v_cache device caches, read and written
 * The block receiving a row's new token must not appear in another row's
 * table (copy on write), as the builder guarantees. Other arguments, errors
 * and the workspace as for pda_paged_decode_attn. */
int32_t pda_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache,
                        void* v_cache, const int32_t* block_table, const int32_t* context_lens,
                        float scale, void* out, const pda_attn_desc* d, void* workspace,
                        size_t ws_bytes, void* stream);

/* Fused decode step on an 8-bit cache: the new rows (d->new_dtype F32 or
 * BF16) are encoded with their destination block's scales exactly as
 * pda_kv_append_quant encodes them, then attended as in
 * pda_paged_decode_attn_quant. */
int32_t pda_decode_step_quant(const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, const float* k_scale,
                              const float* v_scale, const int32_t* block_table,
                              const int32_t* context_lens, float scale, void* out,
                              const pda_attn_desc* d, void* workspace, size_t ws_bytes,
                              void* stream);

/* Paged decode attention with a shared prefix read once  [SoK paper
 * section 2.6: prefix sharing stores a prompt prefix's KV state once for
 * every request that shares it; section 2.5: shared blocks are copy on
 * write]. Many rows start with the same physical blocks (a system prompt);
 * instead of every row reading them, one pass reads each shared block once
 * and applies it to the queries of all rows that share it, the rest of each
 * row is streamed as in pda_paged_decode_attn, and the partial results are
 * merged by log-sum-exp. The result is the attention of each row over all its
 * positions, as pda_paged_decode_attn(_quant) defines it, where logical block
 * i of row b is
 *   prefix_table[i]          for i < prefix_lens[b]
 *   block_table[b][i]        otherwise
 * (block_table[b][i] is never read for i < prefix_lens[b]).
 *   k_scale, v_scale   device [num_blocks][n_kv] fp32 for kv_dtype FP8_E4M3 /
 *                      INT8 (as in pda_paged_decode_attn_quant); NULL for BF16
 *   prefix_table       device int32 [d->prefix_blocks], physical block ids
 *   prefix_lens        device int32 [B], shared-prefix blocks of each row
 * kv_dtype BF16, FP8_E4M3 or INT8; window must be 0; d->prefix_blocks > 0.
 * A row with n > 0 needs 0 <= prefix_lens[b] <= min(prefix_blocks,
 * ceil(n / bs) - 1): the block holding its newest position is its own (copy
 * on write); otherwise, or with an unmapped prefix_table entry among its
 * first prefix_lens[b], the row's output is NaN. Rows with n == 0 are zero
 * (prefix_lens ignored). Other arguments, errors and the workspace
 * (pda_attn_workspace_size of the same descriptor) as for
 * pda_paged_decode_attn. */
int32_t pda_paged_decode_attn_prefix(const void* q, const void* k_cache, const void* v_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_table, const int32_t* context_lens,
                                     const int32_t* prefix_table, const int32_t* prefix_lens,
                                     float scale, void* out, const pda_attn_desc* d,
                                     void* workspace, size_t ws_bytes, void* stream);

/* Fused decode step with a shared prefix read once: each row's new token is
 * written to position n - 1 (as pda_decode_step / pda_decode_step_quant
 * write it; that block is never a prefix block) and the row is then attended
 * as in pda_paged_decode_attn_prefix. The caches end bit for bit as after
 * pda_kv_append(_quant). */
int32_t pda_decode_step_prefix(const void* q, const void* k_new, const void* v_new,
                               void* k_cache, void* v_cache, const float* k_scale,
                               const float* v_scale, const int32_t* block_table,
                               const int32_t* context_lens, const int32_t* prefix_table,
                               const int32_t* prefix_lens, float scale, void* out,
                               const pda_attn_desc* d, void* workspace, size_t ws_bytes,
                               void* stream);

/* 4-bit KV cache with a full-precision residual window  [SoK paper section
 * 2.3: keys quantized per channel and values per token, the most recent
 * tokens held at full precision; section 4.3: 4-bit storage is near-free
 * with per-channel keys; kv-cache tag page, KV-cache quantization teaser:
 * entries are encoded when stored and reconstructed when attention reads
 * them]. Storage (d = d_h, NB = num_blocks):
 *   k_q, v_q   device uint8 [NB][n_kv][16][d/2]: 4-bit codes c in [-7, 7],
 *              stored as the nibble c + 8; in each group of 8 channels
 *              8k .. 8k+7, byte 4k + i holds channel 8k + i in its low nibble
 *              and channel 8k + 4 + i in its high nibble
 *   k_scale    device fp32 [n_kv][d]: key value = k_scale[j][ch] * c, one
 *              fixed scale per (KV head, channel), chosen by the caller
 *   v_scale    device fp32 [NB][n_kv][16]: value = v_scale[pb][j][t] * c, one
 *              scale per token, set when its block is encoded
 *   k_res, v_res device bf16 [B][n_kv][16][d]: each row's open block (its
 *              newest n % 16 tokens) at full precision, token t at slot t % 16
 * A row of n tokens keeps floor(n / 16) encoded blocks and n % 16 residual
 * tokens. */

/* Append of each row's newest token under that policy: for every row b with
 * n = context_lens[b] > 0 (n counts the new token) and every KV head j, the
 * residual slot (n - 1) % 16 of row b receives k_new[b][j][:] / v_new[b][j][:]
 * (bit copy); when that fills the block ((n - 1) % 16 == 15) its 16 tokens
 * are encoded into physical block block_table[b][(n - 1) / 16]:
 *   keys:   c = RNE(x * fp32(1 / k_scale[j][ch])), clamped to [-7, 7]
 *   values: s = fp32(amax_ch |x| / 7) (1 if the amax is 0 or not finite),
 *           c = RNE(x * fp32(1 / s)), clamped; v_scale[pb][j][t] = s
 * k_new, v_new device bf16 [B][n_kv][d]. Descriptor: B, n_kv, d_h,
 * block_size, max_blocks_per_seq, num_blocks, kv_dtype = PDA_INT4; rows with
 * n <= 0 or n > max_blocks_per_seq * 16 append nothing; a block to encode
 * that is unmapped (outside [0, num_blocks)) is skipped, the residual copy
 * is still made. Errors: EINVAL, EHIP. */
int32_t pda_kv_append_int4(const void* k_new, const void* v_new, const int32_t* block_table,
                           const int32_t* context_lens, void* k_q, void* v_q,
                           const float* k_scale, float* v_scale, void* k_res, void* v_res,
                           const pda_attn_desc* d, void* stream);

/* Paged decode attention over that cache: as pda_paged_decode_attn, with
 * row b's positions t < 16 * floor(n / 16) read from its encoded blocks
 * (decoded as above) and the rest from its residual buffer. kv_dtype =
 * PDA_INT4, q bf16 or fp32, window 0. The workspace is required
 * (pda_attn_workspace_size of the same descriptor). Row semantics and
 * errors as for pda_paged_decode_attn. */
int32_t pda_paged_decode_attn_int4(const void* q, const void* k_q, const void* v_q,
                                   const float* k_scale, const float* v_scale,
                                   const void* k_res, const void* v_res,
                                   const int32_t* block_table, const int32_t* context_lens,
                                   float scale, void* out, const pda_attn_desc* d,
                                   void* workspace, size_t ws_bytes, void* stream);

/* One fused decode step over that cache: the append of
 * pda_kv_append_int4 and the attention of pda_paged_decode_attn_int4 in one
 * call, with context_lens counting the new token. The waves that stream a
 * row's blocks also do its append (the residual copy, and the encoding of a
 * block the new token completes, before they read it), so the cache,
 * v_scale, the residual buffers and out hold the same bits as the append
 * followed by the attention. k_new, v_new device bf16 [B][n_kv][d]
 * (new_dtype = PDA_BF16); every other argument, the workspace and the
 * errors as for those two calls. */
int32_t pda_decode_step_int4(const void* q, const void* k_new, const void* v_new, void* k_q,
                             void* v_q, const float* k_scale, float* v_scale, void* k_res,
                             void* v_res, const int32_t* block_table,
                             const int32_t* context_lens, float scale, void* out,
                             const pda_attn_desc* d, void* workspace, size_t ws_bytes,
                             void* stream);

/* Log-sum-exp merge of split-KV partial results. For each of `rows` rows and
 * P partials with (o_p, m_p, l_p):
 *   o_p  part_o[row][p][d_h]  the partial output, normalised over its tokens
 *   m_p  part_ml[row][p][0]   max over its tokens of s_t * log2(e)
 *   l_p  part_ml[row][p][1]   sum over its tokens of 2^(s_t*log2(e) - m_p)
 * out[row] = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - max_p m_p);
 * partials with l_p == 0 are empty and skipped; a row with no live partial
 * is zero. Used inside pda_paged_decode_attn, and exported so partials from
 * several devices holding disjoint token ranges of one sequence (context
 * parallelism, section 9.7) can be merged.
 *   part_o, part_ml, out device; out float [rows][d_h] (d_h 64 or 128);
 *   part_o and out 16-byte aligned, part_ml 8-byte aligned (else EINVAL). */
int32_t pda_lse_merge(const float* part_o, const float* part_ml, int32_t rows, int32_t P,
                      int32_t d_h, float* out, void* stream);

/* ------------------------------------------------------ measurement probe
 * Read-only HBM probe: the bandwidth plain loads reach on this device, the
 * practical ceiling beside the vendor peak for a path that is bound by
 * reading the cache ("9 Decode and KV Cache", section 9.8: bytes moved over
 * elapsed time against the sustained bandwidth). Not part of the method.
 *   buf           device, 16-byte aligned, `bytes` long (read only).
 *   tile_offsets  NULL: sequential mode. `waves` waves walk buf in 4 KiB
 *                 steps, wave w reading bytes [(s * waves + w) * 4096, +4096)
 *                 of step s, for floor(bytes / 4096 / waves) steps.
 *                 Otherwise device int64 [n_tiles]: tile mode. Tile i is the
 *                 `tile_bytes` bytes at buf + tile_offsets[i]; wave w reads
 *                 tiles [w * n_tiles / waves, (w + 1) * n_tiles / waves) in
 *                 order with four tiles in flight. The caller guarantees that
 *                 every offset is a multiple of 16 and offset + tile_bytes <=
 *                 bytes (device data is not inspected).
 *   tile_bytes    1024, 2048, 4096 or 8192 (tile mode).
 *   waves         multiple of 4 in [4, 65536]: 64-lane waves, four per
 *                 workgroup.
 *   sink          device uint32 [waves * 64]: a checksum of every dword read
 *                 (so no load is elided), overwritten.
 * Loads are 16 bytes per lane and non-temporal, like the attention
 * kernels' cache loads. EINVAL on a NULL buffer, bad sizes or alignment. */
int32_t pda_hbm_read_probe(const void* buf, size_t bytes, const int64_t* tile_offsets,
                           int64_t n_tiles, int32_t tile_bytes, int32_t waves, uint32_t* sink,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PDA_H */
