// Host block manager: fixed-size blocks from one shared pool, chained-hash
// prefix sharing and LRU reuse of unreferenced cached blocks.
//
// TensorSharp "高级功能" page, section "连续批处理与分页 KV 缓存" (paged KV pool;
// block-hash prefix sharing across concurrent and sequential requests) and
// section "内存优化" (paged KV block pool with LRU eviction and cross-session
// content-hash reuse). The exact policy is spelled out at kv_pool_alloc in
// pagedkv.h; this file implements it with O(1) free-list operations.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "status.h"

namespace pkv {

static thread_local std::string g_last_error;

void set_error(const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
}

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

inline uint64_t fnv_byte(uint64_t h, uint8_t b) { return (h ^ b) * kFnvPrime; }

// FNV-1a-64 over (parent hash, 8 bytes little-endian) || tokens (int32 little-endian).
uint64_t chain_hash(uint64_t parent, const int32_t *tok, int n) {
    uint64_t h = kFnvOffset;
    for (int i = 0; i < 8; ++i) h = fnv_byte(h, uint8_t(parent >> (8 * i)));
    for (int t = 0; t < n; ++t) {
        uint32_t u = uint32_t(tok[t]);
        for (int i = 0; i < 4; ++i) h = fnv_byte(h, uint8_t(u >> (8 * i)));
    }
    return h;
}

struct Entry {
    int32_t block;
    int32_t parent;       // -1 for the first block of a sequence
    uint32_t parent_gen;  // reuse generation of the parent when registered
    std::vector<int32_t> tokens;
};

struct Seq {
    std::vector<int32_t> tokens;
    std::vector<int32_t> blocks;   // -1 for blocks freed by kv_pool_drop_prefix
    std::vector<uint64_t> hashes;  // one per full block
    bool dropped = false;          // some block was freed: no sharing from here on
};

}  // namespace
}  // namespace pkv

struct kv_pool {
    int32_t n = 0, B = 0;
    // FIFO free list as a doubly linked list over block ids (-1 terminated).
    std::vector<int32_t> prev, next;
    int32_t head = -1, tail = -1, free_count = 0;
    std::vector<uint8_t> in_free;
    std::vector<int32_t> ref;
    std::vector<uint32_t> gen;
    std::vector<uint8_t> has_hash;
    std::vector<uint64_t> blk_hash;
    std::unordered_map<uint64_t, pkv::Entry> table;
    std::unordered_map<int64_t, pkv::Seq> seqs;
    uint64_t hash_mask = ~0ull;  // test hook: forces collisions when narrowed

    void push_back(int32_t b) {
        prev[b] = tail;
        next[b] = -1;
        if (tail >= 0) next[tail] = b; else head = b;
        tail = b;
        in_free[b] = 1;
        ++free_count;
    }
    void unlink(int32_t b) {
        if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
        if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
        prev[b] = next[b] = -1;
        in_free[b] = 0;
        --free_count;
    }
    int32_t pop() {
        int32_t b = head;
        unlink(b);
        if (has_hash[b]) {
            table.erase(blk_hash[b]);
            has_hash[b] = 0;
        }
        ++gen[b];
        ref[b] = 1;
        return b;
    }
    uint64_t hash(uint64_t parent, const int32_t *tok) const {
        return pkv::chain_hash(parent, tok, B) & hash_mask;
    }
    void reg(int32_t b, uint64_t h, int32_t parent, const int32_t *tok) {
        if (table.count(h)) return;
        pkv::Entry e;
        e.block = b;
        e.parent = parent;
        e.parent_gen = parent >= 0 ? gen[parent] : 0u;
        e.tokens.assign(tok, tok + B);
        table.emplace(h, std::move(e));
        has_hash[b] = 1;
        blk_hash[b] = h;
    }
};

extern "C" {

int kv_abi_version(void) { return PAGEDKV_ABI_VERSION; }

const char *kv_last_error(void) { return pkv::g_last_error.c_str(); }

int kv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t *initial_free_order,
                   kv_pool **out) {
    try {
        if (!out) PKV_FAIL(KV_EINVAL, "kv_pool_create: out is NULL");
        if (num_blocks <= 0 || block_size <= 0)
            PKV_FAIL(KV_EINVAL, "kv_pool_create: num_blocks (%d) and block_size (%d) must be positive",
                     num_blocks, block_size);
        std::vector<int32_t> order(num_blocks);
        if (initial_free_order) {
            std::vector<uint8_t> seen(num_blocks, 0);
            for (int32_t i = 0; i < num_blocks; ++i) {
                int32_t b = initial_free_order[i];
                if (b < 0 || b >= num_blocks || seen[b])
                    PKV_FAIL(KV_EINVAL, "kv_pool_create: initial_free_order is not a permutation of 0..%d",
                             num_blocks - 1);
                seen[b] = 1;
                order[i] = b;
            }
        } else {
            for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
        }
        kv_pool *p = new kv_pool;
        p->n = num_blocks;
        p->B = block_size;
        p->prev.assign(num_blocks, -1);
        p->next.assign(num_blocks, -1);
        p->in_free.assign(num_blocks, 0);
        p->ref.assign(num_blocks, 0);
        p->gen.assign(num_blocks, 0);
        p->has_hash.assign(num_blocks, 0);
        p->blk_hash.assign(num_blocks, 0);
        for (int32_t b : order) p->push_back(b);
        *out = p;
        return KV_OK;
    } catch (const std::bad_alloc &) {
        PKV_FAIL(KV_EINTERNAL, "kv_pool_create: host allocation failed");
    } catch (...) {
        PKV_FAIL(KV_EINTERNAL, "kv_pool_create: unexpected exception");
    }
}

void kv_pool_destroy(kv_pool *pool) { delete pool; }

int kv_pool_alloc(kv_pool *pool, int64_t seq_id, const int32_t *new_token_ids, int32_t n_new,
                  int32_t *block_table_row, int32_t max_blocks, int32_t *num_blocks,
                  int32_t *context_len, int32_t *slot_mapping) {
    try {
        if (!pool) PKV_FAIL(KV_EINVAL, "kv_pool_alloc: pool is NULL");
        if (n_new < 0) PKV_FAIL(KV_EINVAL, "kv_pool_alloc: n_new (%d) < 0", n_new);
        if (n_new > 0 && (!new_token_ids || !slot_mapping))
            PKV_FAIL(KV_EINVAL, "kv_pool_alloc: token ids or slot_mapping is NULL");
        if (!block_table_row || max_blocks < 0)
            PKV_FAIL(KV_EINVAL, "kv_pool_alloc: block_table_row is NULL or max_blocks < 0");
        const int32_t B = pool->B;
        auto it = pool->seqs.find(seq_id);
        static const pkv::Seq kEmpty;
        const pkv::Seq &cur = it == pool->seqs.end() ? kEmpty : it->second;
        const int64_t n0 = int64_t(cur.tokens.size());
        const int64_t n1 = n0 + n_new;
        const int64_t nb0 = (n0 + B - 1) / B;
        const int64_t nb1 = (n1 + B - 1) / B;
        if (n1 > INT32_MAX) PKV_FAIL(KV_EINVAL, "kv_pool_alloc: context length overflows int32");
        if (nb1 > max_blocks)
            PKV_FAIL(KV_EINVAL, "kv_pool_alloc: sequence %lld needs %lld blocks, max_blocks is %d",
                     (long long)seq_id, (long long)nb1, max_blocks);

        std::vector<int32_t> all(cur.tokens);
        all.insert(all.end(), new_token_ids, new_token_ids + n_new);

        // Phase 1 (read only): the run of shared blocks starting at a block boundary.
        struct Hit { int32_t block; uint64_t hash; };
        std::vector<Hit> hits;
        if (n0 % B == 0 && !cur.dropped) {
            uint64_t ph = cur.hashes.empty() ? 0 : cur.hashes.back();
            int32_t parent = cur.blocks.empty() ? -1 : cur.blocks.back();
            for (int64_t j = nb0; j < nb1; ++j) {
                if ((j + 1) * B > n1) break;
                const int32_t *tok = all.data() + j * B;
                uint64_t h = pool->hash(ph, tok);
                auto e = pool->table.find(h);
                if (e == pool->table.end()) break;
                const pkv::Entry &en = e->second;
                uint32_t want_gen = parent >= 0 ? pool->gen[parent] : 0u;
                if (en.parent != parent || en.parent_gen != want_gen ||
                    std::memcmp(en.tokens.data(), tok, sizeof(int32_t) * B) != 0)
                    break;
                hits.push_back({en.block, h});
                ph = h;
                parent = en.block;
            }
        }
        int64_t revive = 0;
        for (const Hit &h : hits) revive += pool->in_free[h.block];
        const int64_t n_pop = (nb1 - nb0) - int64_t(hits.size());
        if (n_pop > pool->free_count - revive)
            PKV_FAIL(KV_ENOMEM, "kv_pool_alloc: sequence %lld needs %lld new blocks, %lld free",
                     (long long)seq_id, (long long)n_pop, (long long)(pool->free_count - revive));

        // Phase 2: commit (nothing below can fail except host allocation).
        pkv::Seq &st = pool->seqs[seq_id];
        int32_t w = 0;  // slot_mapping cursor
        if (n0 % B) {
            const int32_t b = st.blocks.back();
            const int64_t off = n0 % B;
            const int64_t take = std::min<int64_t>(B - off, n_new);
            for (int64_t i = 0; i < take; ++i) slot_mapping[w++] = int32_t(b * B + off + i);
            if (off + take == B) {
                const int64_t j = nb0 - 1;
                const uint64_t ph = st.hashes.empty() ? 0 : st.hashes.back();
                const uint64_t h = pool->hash(ph, all.data() + j * B);
                st.hashes.push_back(h);
                if (!st.dropped) pool->reg(b, h, j > 0 ? st.blocks[j - 1] : -1, all.data() + j * B);
            }
        }
        for (const Hit &h : hits) {
            if (pool->in_free[h.block]) pool->unlink(h.block);
            ++pool->ref[h.block];
            st.blocks.push_back(h.block);
            st.hashes.push_back(h.hash);
            for (int32_t i = 0; i < B; ++i) slot_mapping[w++] = -1;
        }
        for (int64_t j = nb0 + int64_t(hits.size()); j < nb1; ++j) {
            const int32_t b = pool->pop();
            const int64_t first = std::max<int64_t>(n0, j * B);
            const int64_t last = std::min<int64_t>(n1, (j + 1) * B);
            for (int64_t t = first; t < last; ++t) slot_mapping[w++] = int32_t(b * B + (t - j * B));
            const int32_t parent = st.blocks.empty() ? -1 : st.blocks.back();
            st.blocks.push_back(b);
            if (last - j * B == B) {
                const uint64_t ph = st.hashes.empty() ? 0 : st.hashes.back();
                const uint64_t h = pool->hash(ph, all.data() + j * B);
                st.hashes.push_back(h);
                if (!st.dropped) pool->reg(b, h, parent, all.data() + j * B);
            }
        }
        st.tokens.swap(all);
        for (int32_t j = 0; j < max_blocks; ++j)
            block_table_row[j] = j < int32_t(st.blocks.size()) ? st.blocks[j] : -1;
        if (num_blocks) *num_blocks = int32_t(st.blocks.size());
        if (context_len) *context_len = int32_t(n1);
        return KV_OK;
    } catch (const std::bad_alloc &) {
        PKV_FAIL(KV_EINTERNAL, "kv_pool_alloc: host allocation failed");
    } catch (...) {
        PKV_FAIL(KV_EINTERNAL, "kv_pool_alloc: unexpected exception");
    }
}

int kv_pool_release(kv_pool *pool, int64_t seq_id) {
    try {
        if (!pool) PKV_FAIL(KV_EINVAL, "kv_pool_release: pool is NULL");
        auto it = pool->seqs.find(seq_id);
        if (it == pool->seqs.end())
            PKV_FAIL(KV_EINVAL, "kv_pool_release: unknown sequence %lld", (long long)seq_id);
        const std::vector<int32_t> &bl = it->second.blocks;
        for (auto b = bl.rbegin(); b != bl.rend(); ++b)
            if (*b >= 0 && --pool->ref[*b] == 0) pool->push_back(*b);
        pool->seqs.erase(it);
        return KV_OK;
    } catch (...) {
        PKV_FAIL(KV_EINTERNAL, "kv_pool_release: unexpected exception");
    }
}

int kv_pool_truncate(kv_pool *pool, int64_t seq_id, int32_t new_len, int32_t *copy_src, int32_t *copy_dst) {
    try {
        if (!pool || !copy_src || !copy_dst) PKV_FAIL(KV_EINVAL, "kv_pool_truncate: pool or an output is NULL");
        auto it = pool->seqs.find(seq_id);
        if (it == pool->seqs.end())
            PKV_FAIL(KV_EINVAL, "kv_pool_truncate: unknown sequence %lld", (long long)seq_id);
        pkv::Seq &st = it->second;
        const int64_t n = int64_t(st.tokens.size());
        if (new_len < 0 || new_len > n)
            PKV_FAIL(KV_EINVAL, "kv_pool_truncate: new_len %d outside 0 .. %lld", new_len, (long long)n);
        const int32_t B = pool->B;
        const int64_t nb = int64_t(st.blocks.size());
        const int64_t keep = (int64_t(new_len) + B - 1) / B;
        // the new last block was full: its later slots will be written again
        const bool tail_full = new_len % B != 0 && int64_t(st.hashes.size()) >= keep;
        const int32_t tail = tail_full ? st.blocks[keep - 1] : -1;
        if (tail_full && tail < 0)
            PKV_FAIL(KV_EINVAL, "kv_pool_truncate: new_len %d ends inside a dropped block", new_len);
        const bool shared = tail_full && pool->ref[tail] > 1;
        if (shared) {
            int64_t freed = 0;
            for (int64_t j = keep; j < nb; ++j) freed += st.blocks[j] >= 0 && pool->ref[st.blocks[j]] == 1;
            if (pool->free_count + freed < 1)
                PKV_FAIL(KV_ENOMEM, "kv_pool_truncate: a shared block must be copied and no block is free");
        }
        for (int64_t j = nb - 1; j >= keep; --j) {
            const int32_t b = st.blocks[j];
            if (b >= 0 && --pool->ref[b] == 0) pool->push_back(b);
        }
        st.blocks.resize(size_t(keep));
        st.hashes.resize(size_t(new_len / B));
        st.tokens.resize(size_t(new_len));
        *copy_src = *copy_dst = -1;
        if (tail_full) {
            if (shared) {
                --pool->ref[tail];
                const int32_t d = pool->pop();
                st.blocks[size_t(keep - 1)] = d;
                *copy_src = tail;
                *copy_dst = d;
            } else {
                if (pool->has_hash[tail]) {
                    pool->table.erase(pool->blk_hash[tail]);
                    pool->has_hash[tail] = 0;
                }
                ++pool->gen[tail];
            }
        }
        return KV_OK;
    } catch (...) {
        PKV_FAIL(KV_EINTERNAL, "kv_pool_truncate: unexpected exception");
    }
}

int kv_pool_drop_prefix(kv_pool *pool, int64_t seq_id, int32_t first_kept) {
    try {
        if (!pool) PKV_FAIL(KV_EINVAL, "kv_pool_drop_prefix: pool is NULL");
        auto it = pool->seqs.find(seq_id);
        if (it == pool->seqs.end())
            PKV_FAIL(KV_EINVAL, "kv_pool_drop_prefix: unknown sequence %lld", (long long)seq_id);
        if (first_kept < 0) PKV_FAIL(KV_EINVAL, "kv_pool_drop_prefix: first_kept %d < 0", first_kept);
        pkv::Seq &st = it->second;
        const int64_t upto = std::min<int64_t>(first_kept, int64_t(st.tokens.size())) / pool->B;
        for (int64_t j = upto - 1; j >= 0; --j) {
            const int32_t b = st.blocks[size_t(j)];
            if (b < 0) continue;
            if (--pool->ref[b] == 0) pool->push_back(b);
            st.blocks[size_t(j)] = -1;
            st.dropped = true;
        }
        return KV_OK;
    } catch (...) {
        PKV_FAIL(KV_EINTERNAL, "kv_pool_drop_prefix: unexpected exception");
    }
}

int kv_tree_masks(const int32_t *parents, int32_t n, uint32_t *masks) {
    if (!parents || !masks || n < 0 || n > 32)
        PKV_FAIL(KV_EINVAL, "kv_tree_masks: null pointer or n %d outside 0 .. 32", n);
    uint32_t m[32];
    for (int32_t r = 0; r < n; ++r) {
        const int32_t p = parents[r];
        if (p < -1 || p >= r) PKV_FAIL(KV_EINVAL, "kv_tree_masks: parent %d of row %d is not -1 or an earlier row", p, r);
        m[r] = (1u << r) | (p >= 0 ? m[p] : 0u);
    }
    for (int32_t r = 0; r < n; ++r) masks[r] = m[r];
    return KV_OK;
}

int kv_pool_stats(const kv_pool *pool, int32_t *free_blocks, int32_t *cached_blocks,
                  int32_t *live_blocks) {
    if (!pool) PKV_FAIL(KV_EINVAL, "kv_pool_stats: pool is NULL");
    int32_t cached = 0, live = 0;
    for (int32_t b = pool->head; b >= 0; b = pool->next[b]) cached += pool->has_hash[b];
    for (int32_t r : pool->ref) live += r > 0;
    if (free_blocks) *free_blocks = pool->free_count;
    if (cached_blocks) *cached_blocks = cached;
    if (live_blocks) *live_blocks = live;
    return KV_OK;
}

int kv_pool_set_hash_mask(kv_pool *pool, uint64_t mask) {
    if (!pool) PKV_FAIL(KV_EINVAL, "kv_pool_set_hash_mask: pool is NULL");
    pool->hash_mask = mask;
    return KV_OK;
}

}  // extern "C"
