// pool.cpp -- host KV block manager: fixed-size blocks handed out on demand
// from a free list, per-request block tables, and reference counts so that
// several requests can share a prefix block with copy on write ("9 Decode and
// KV Cache", section 9.5, PagedAttention and its block table; SoK paper
// sections 2.5-2.6). Running out of blocks is reported, never handled here:
// it is the engine's preemption signal (section 9.5).
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pda.h"
#include "pda_internal.h"

struct pda_pool {
    int32_t num_blocks;
    std::deque<int32_t> free_list;   // FIFO: allocate from the front, release to the back
    std::vector<int32_t> ref;        // 0 = free
};

using pda::set_error;

extern "C" int32_t pda_pool_create(int32_t num_blocks, const int32_t* free_order,
                                   pda_pool** out) {
    if (!out || num_blocks <= 0) {
        set_error("pda_pool_create: need out != NULL and num_blocks > 0");
        return PDA_EINVAL;
    }
    *out = nullptr;
    pda_pool* p = new (std::nothrow) pda_pool;
    if (!p) {
        set_error("pda_pool_create: out of host memory");
        return PDA_EINVAL;
    }
    p->num_blocks = num_blocks;
    p->ref.assign((size_t)num_blocks, 0);
    if (free_order) {
        std::vector<char> seen((size_t)num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            const int32_t id = free_order[i];
            if (id < 0 || id >= num_blocks || seen[(size_t)id]) {
                delete p;
                set_error("pda_pool_create: free_order is not a permutation of 0..%d", num_blocks - 1);
                return PDA_EINVAL;
            }
            seen[(size_t)id] = 1;
            p->free_list.push_back(id);
        }
    } else {
        for (int32_t i = 0; i < num_blocks; ++i) p->free_list.push_back(i);
    }
    *out = p;
    return PDA_OK;
}

extern "C" int32_t pda_pool_destroy(pda_pool* pool) {
    delete pool;
    return PDA_OK;
}

extern "C" int32_t pda_pool_alloc(pda_pool* pool, int32_t n, int32_t* ids_out) {
    if (!pool || n < 0 || (n > 0 && !ids_out)) {
        set_error("pda_pool_alloc: bad arguments");
        return PDA_EINVAL;
    }
    if ((size_t)n > pool->free_list.size()) {
        set_error("pda_pool_alloc: %d blocks requested, %zu free", n, pool->free_list.size());
        return PDA_ENOSPC;
    }
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = pool->free_list.front();
        pool->free_list.pop_front();
        pool->ref[(size_t)id] = 1;
        ids_out[i] = id;
    }
    return PDA_OK;
}

extern "C" int32_t pda_pool_share(pda_pool* pool, int32_t n, const int32_t* ids) {
    if (!pool || n < 0 || (n > 0 && !ids)) {
        set_error("pda_pool_share: bad arguments");
        return PDA_EINVAL;
    }
    for (int32_t i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= pool->num_blocks || pool->ref[(size_t)ids[i]] == 0) {
            set_error("pda_pool_share: block %d is not allocated", ids[i]);
            return PDA_EINVAL;
        }
    }
    for (int32_t i = 0; i < n; ++i) ++pool->ref[(size_t)ids[i]];
    return PDA_OK;
}

extern "C" int32_t pda_pool_free(pda_pool* pool, int32_t n, const int32_t* ids) {
    if (!pool || n < 0 || (n > 0 && !ids)) {
        set_error("pda_pool_free: bad arguments");
        return PDA_EINVAL;
    }
    std::unordered_map<int32_t, int32_t> count;
    for (int32_t i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= pool->num_blocks) {
            set_error("pda_pool_free: block id %d out of range", ids[i]);
            return PDA_EINVAL;
        }
        if (++count[ids[i]] > pool->ref[(size_t)ids[i]]) {
            set_error("pda_pool_free: block %d released more often than referenced", ids[i]);
            return PDA_EINVAL;
        }
    }
    for (int32_t i = 0; i < n; ++i) {
        if (--pool->ref[(size_t)ids[i]] == 0) pool->free_list.push_back(ids[i]);
    }
    return PDA_OK;
}

extern "C" int32_t pda_pool_num_free(const pda_pool* pool, int32_t* out) {
    if (!pool || !out) {
        set_error("pda_pool_num_free: bad arguments");
        return PDA_EINVAL;
    }
    *out = (int32_t)pool->free_list.size();
    return PDA_OK;
}

extern "C" int32_t pda_pool_refcount(const pda_pool* pool, int32_t id, int32_t* out) {
    if (!pool || !out || id < 0 || id >= pool->num_blocks) {
        set_error("pda_pool_refcount: bad arguments");
        return PDA_EINVAL;
    }
    *out = pool->ref[(size_t)id];
    return PDA_OK;
}

extern "C" int32_t pda_build_block_table(pda_pool* pool, int32_t B, const int32_t* context_lens,
                                         int32_t block_size, int32_t n_shared,
                                         const int32_t* shared_ids, int32_t max_blocks,
                                         int32_t* block_table_out, int64_t* slot_mapping_out) {
    if (!pool || B < 0 || block_size <= 0 || n_shared < 0 || max_blocks <= 0 ||
        (B > 0 && (!context_lens || !block_table_out || !slot_mapping_out)) ||
        (n_shared > 0 && !shared_ids)) {
        set_error("pda_build_block_table: bad arguments");
        return PDA_EINVAL;
    }
    // plan every row first: all-or-nothing
    std::vector<int32_t> nblk((size_t)B), nsh((size_t)B);
    int64_t fresh = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t n = context_lens[b];
        if (n < 0) {
            set_error("pda_build_block_table: row %d has negative length", b);
            return PDA_EINVAL;
        }
        const int64_t blocks = ((int64_t)n + block_size - 1) / block_size;
        if (blocks > max_blocks) {
            set_error("pda_build_block_table: row %d needs %lld blocks, table holds %d", b,
                      (long long)blocks, max_blocks);
            return PDA_EINVAL;
        }
        nblk[(size_t)b] = (int32_t)blocks;
        // the block that receives the newest token is private (copy on write)
        const int32_t sh = blocks > 0 ? (int32_t)std::min<int64_t>(n_shared, blocks - 1) : 0;
        nsh[(size_t)b] = sh;
        fresh += blocks - sh;
    }
    for (int32_t i = 0; i < n_shared; ++i) {
        const int32_t id = shared_ids[i];
        if (id < 0 || id >= pool->num_blocks || pool->ref[(size_t)id] == 0) {
            set_error("pda_build_block_table: shared block %d is not allocated", id);
            return PDA_EINVAL;
        }
    }
    if (fresh > (int64_t)pool->free_list.size()) {
        set_error("pda_build_block_table: %lld fresh blocks needed, %zu free", (long long)fresh,
                  pool->free_list.size());
        return PDA_ENOSPC;
    }
    for (int32_t b = 0; b < B; ++b) {
        int32_t* row = block_table_out + (int64_t)b * max_blocks;
        const int32_t sh = nsh[(size_t)b], blocks = nblk[(size_t)b];
        for (int32_t i = 0; i < sh; ++i) {
            row[i] = shared_ids[i];
            ++pool->ref[(size_t)shared_ids[i]];
        }
        for (int32_t i = sh; i < blocks; ++i) {
            const int32_t id = pool->free_list.front();
            pool->free_list.pop_front();
            pool->ref[(size_t)id] = 1;
            row[i] = id;
        }
        for (int32_t i = blocks; i < max_blocks; ++i) row[i] = -1;
        const int32_t n = context_lens[b];
        slot_mapping_out[b] = n > 0 ? (int64_t)row[(n - 1) / block_size] * block_size +
                                          (n - 1) % block_size
                                    : -1;
    }
    return PDA_OK;
}
