// Host-side block pool of the block table: free list plus reference counts
// (declared in ps.h).  Plain C++, no device calls.
#include <cstdint>
#include <new>
#include <set>
#include <vector>

#include "../../include/ps.h"

struct ps_block_pool {
    std::vector<int32_t> refs;  // references per block, 0 = free
    std::set<int32_t> free;     // free blocks, lowest first
};

namespace {
bool in_range(const ps_block_pool* p, int32_t b) { return p && b >= 0 && b < (int32_t)p->refs.size(); }
}  // namespace

extern "C" {

int ps_block_pool_create(int32_t n_blocks, ps_block_pool** out) {
    if (!out) return PS_ERR_INVALID;
    *out = nullptr;
    if (n_blocks < 1) return PS_ERR_INVALID;
    ps_block_pool* p = new (std::nothrow) ps_block_pool;
    if (!p) return PS_ERR_CAPACITY;
    try {
        p->refs.assign((size_t)n_blocks, 0);
        for (int32_t b = 0; b < n_blocks; ++b) p->free.insert(p->free.end(), b);
    } catch (...) {
        delete p;
        return PS_ERR_CAPACITY;
    }
    *out = p;
    return PS_OK;
}

int ps_block_pool_destroy(ps_block_pool* pool) {
    delete pool;
    return PS_OK;
}

int ps_block_alloc(ps_block_pool* pool, int32_t* block) {
    if (!pool || !block) return PS_ERR_INVALID;
    if (pool->free.empty()) return PS_ERR_CAPACITY;
    const int32_t b = *pool->free.begin();
    pool->free.erase(pool->free.begin());
    pool->refs[(size_t)b] = 1;
    *block = b;
    return PS_OK;
}

int ps_block_retain(ps_block_pool* pool, int32_t block) {
    if (!in_range(pool, block) || pool->refs[(size_t)block] == 0) return PS_ERR_INVALID;
    if (pool->refs[(size_t)block] == INT32_MAX) return PS_ERR_CAPACITY;
    ++pool->refs[(size_t)block];
    return PS_OK;
}

int ps_block_release(ps_block_pool* pool, int32_t block) {
    if (!in_range(pool, block) || pool->refs[(size_t)block] == 0) return PS_ERR_INVALID;
    if (--pool->refs[(size_t)block] == 0) {
        try {
            pool->free.insert(block);
        } catch (...) {
            ++pool->refs[(size_t)block];
            return PS_ERR_CAPACITY;
        }
    }
    return PS_OK;
}

int ps_block_refcount(const ps_block_pool* pool, int32_t block, int32_t* count) {
    if (!in_range(pool, block) || !count) return PS_ERR_INVALID;
    *count = pool->refs[(size_t)block];
    return PS_OK;
}

int ps_block_free_count(const ps_block_pool* pool, int32_t* count) {
    if (!pool || !count) return PS_ERR_INVALID;
    *count = (int32_t)pool->free.size();
    return PS_OK;
}

}  // extern "C"
