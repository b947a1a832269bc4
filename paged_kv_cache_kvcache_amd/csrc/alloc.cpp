// Host block manager: the block tables, slot mappings and prefix reuse behind the paged KV cache.
//
// Blocks of 256 tokens come from a FIFO free pool (intelliparadigm.com Nano-vLLM article, §2.1
// 动态分块内存管理), are shared by reference count ("1200行代码挑战vLLM", §2 内存管理策略), and full
// prompt blocks are found again through a chained hash of the prompt prefix ("1200行代码挑战vLLM",
// §性能优化 1. 前缀缓存).  Released blocks keep their hash and contents until reused (lazy release,
// intelliparadigm.com article, §7.2 关键优化点).  The exact rules are listed in pkv.h.
//
// Data structures are chosen for O(1) steps without heap traffic in the steady state: the free
// deque is an intrusive doubly linked list over block ids (a hit on a released block unlinks it
// from the middle), the prefix table is a hash map from the 64-bit chained hash to the block that
// last registered it, sequences live in a slab of reusable records found through an
// open-addressing index, the tokens of a partially filled block are kept with the block (a fork
// copies no tokens), and the batch calls' dry runs mark sequences and blocks with an epoch stamp
// instead of building maps.
#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pkv_internal.h"

using pkv::fail;
using pkv::kBlock;

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

inline uint64_t fnv_byte(uint64_t h, uint8_t b) { return (h ^ b) * kFnvPrime; }

// FNV-1a-64 over le64(prev) followed by le32 of each of the 256 tokens.
uint64_t chained_block_hash(uint64_t prev, const int32_t* toks) {
    uint64_t h = kFnvOffset;
    for (int i = 0; i < 8; ++i) h = fnv_byte(h, uint8_t(prev >> (8 * i)));
    for (int t = 0; t < kBlock; ++t) {
        uint32_t u = uint32_t(toks[t]);
        for (int i = 0; i < 4; ++i) h = fnv_byte(h, uint8_t(u >> (8 * i)));
    }
    return h;
}

struct Seq {
    std::vector<int32_t> blocks;  // capacity kept when the record is reused
    int32_t len = 0;              // tokens held
    int32_t n_cached = 0;
    uint64_t last_hash = 0;  // hash of the last full block (chain input for the next one)
    // dry-run state of the batch call that set stamp
    uint32_t stamp = 0;
    int32_t dry_len = 0;
    int32_t dry_last = 0;
};

// Sequence id -> slab slot: linear probing, load factor at most 1/2, deletion by backward shift
// (no tombstones).
class SeqIndex {
    struct Entry {
        int64_t key;
        int32_t slot;  // < 0: empty
    };
    std::vector<Entry> t_;
    size_t mask_ = 0, n_ = 0;

    static uint64_t mix(int64_t k) {  // splitmix64 finaliser
        uint64_t z = uint64_t(k) + 0x9e3779b97f4a7c15ull;
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    }
    void grow() {
        std::vector<Entry> old = std::move(t_);
        t_.assign(old.empty() ? 64 : old.size() * 2, Entry{0, -1});
        mask_ = t_.size() - 1;
        for (const Entry& e : old)
            if (e.slot >= 0) {
                size_t i = mix(e.key) & mask_;
                while (t_[i].slot >= 0) i = (i + 1) & mask_;
                t_[i] = e;
            }
    }

public:
    int32_t find(int64_t key) const {
        if (t_.empty()) return -1;
        for (size_t i = mix(key) & mask_;; i = (i + 1) & mask_) {
            if (t_[i].slot < 0) return -1;
            if (t_[i].key == key) return t_[i].slot;
        }
    }
    void insert(int64_t key, int32_t slot) {  // key not present
        if (2 * (n_ + 1) > t_.size()) grow();
        size_t i = mix(key) & mask_;
        while (t_[i].slot >= 0) i = (i + 1) & mask_;
        t_[i] = Entry{key, slot};
        ++n_;
    }
    int32_t erase(int64_t key) {  // the slot key mapped to, or -1
        if (t_.empty()) return -1;
        size_t i = mix(key) & mask_;
        while (t_[i].slot >= 0 && t_[i].key != key) i = (i + 1) & mask_;
        if (t_[i].slot < 0) return -1;
        const int32_t slot = t_[i].slot;
        // shift back every later entry of the run whose home is not in (i, j]
        for (size_t j = (i + 1) & mask_; t_[j].slot >= 0; j = (j + 1) & mask_) {
            const size_t home = mix(t_[j].key) & mask_;
            if (((j - home) & mask_) >= ((j - i) & mask_)) {
                t_[i] = t_[j];
                i = j;
            }
        }
        t_[i].slot = -1;
        --n_;
        return slot;
    }
};

}  // namespace

struct pkv_allocator {
    int32_t nblocks = 0;
    bool prefix = true;
    bool const_hash = false;
    uint64_t const_hash_value = 0;

    // free deque: intrusive list, -1 terminated
    std::vector<int32_t> nxt, prv;
    std::vector<uint8_t> in_free;
    int32_t head = -1, tail = -1, nfree = 0;

    std::vector<int32_t> ref;
    std::vector<uint8_t> has_hash;
    std::vector<uint64_t> bhash;
    // tokens of a block: all 256 of a registered (hashed) block, the rows in use of a partially
    // filled one (its holders are all at the same length: an append to a shared partial block
    // copies it first)
    std::vector<std::vector<int32_t>> btok;
    std::unordered_map<uint64_t, int32_t> table;

    // sequences: records in a slab (stable addresses), reused through a free list
    std::deque<Seq> slab;
    std::vector<int32_t> free_slots;
    SeqIndex index;

    // batch dry runs: a stamp per sequence record (in Seq) and per block
    uint32_t epoch = 0;
    std::vector<uint32_t> blk_stamp;
    std::vector<int32_t> blk_dry_ref;
    std::vector<std::pair<int64_t, int32_t>> id_scratch;

    Seq* find(int64_t id) {
        const int32_t k = index.find(id);
        return k < 0 ? nullptr : &slab[size_t(k)];
    }
    const Seq* find(int64_t id) const {
        const int32_t k = index.find(id);
        return k < 0 ? nullptr : &slab[size_t(k)];
    }
    Seq& admit(int64_t id) {  // id not present; the record comes back empty
        int32_t k;
        if (!free_slots.empty()) {
            k = free_slots.back();
            free_slots.pop_back();
        } else {
            k = int32_t(slab.size());
            slab.emplace_back();
        }
        Seq& s = slab[size_t(k)];
        s.blocks.clear();
        s.len = s.n_cached = 0;
        s.last_hash = 0;
        index.insert(id, k);
        return s;
    }
    void release(int64_t id) {
        const int32_t k = index.erase(id);
        if (k >= 0) free_slots.push_back(k);
    }
    uint32_t next_epoch() {  // a stamp no record or block holds
        if (++epoch == 0) {
            for (Seq& q : slab) q.stamp = 0;
            std::fill(blk_stamp.begin(), blk_stamp.end(), 0u);
            epoch = 1;
        }
        return epoch;
    }

    uint64_t hash_block(uint64_t prev, const int32_t* toks) const {
        return const_hash ? const_hash_value : chained_block_hash(prev, toks);
    }

    void push_back(int32_t b) {
        nxt[b] = -1;
        prv[b] = tail;
        if (tail >= 0) nxt[tail] = b; else head = b;
        tail = b;
        in_free[b] = 1;
        ++nfree;
    }
    void unlink(int32_t b) {
        if (prv[b] >= 0) nxt[prv[b]] = nxt[b]; else head = nxt[b];
        if (nxt[b] >= 0) prv[nxt[b]] = prv[b]; else tail = prv[b];
        nxt[b] = prv[b] = -1;
        in_free[b] = 0;
        --nfree;
    }
    // Head of the free deque, wiped of its previous identity, with one reference.
    int32_t pop_fresh() {
        int32_t b = head;
        unlink(b);
        if (has_hash[b]) {
            auto it = table.find(bhash[b]);
            if (it != table.end() && it->second == b) table.erase(it);
        }
        has_hash[b] = 0;
        bhash[b] = 0;
        btok[b].clear();
        ref[b] = 1;
        return b;
    }
    void register_block(int32_t b, uint64_t h, const int32_t* toks) {
        if (toks != nullptr) btok[b].assign(toks, toks + kBlock);
        has_hash[b] = 1;
        bhash[b] = h;
        table[h] = b;
    }
};

extern "C" {

int pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_order,
                     int32_t prefix_cache, pkv_allocator** out) {
    PKV_REQUIRE(out != nullptr, PKV_ERR_INVALID, "out is NULL");
    *out = nullptr;
    PKV_REQUIRE(block_size == kBlock, PKV_ERR_UNSUPPORTED, "block_size %d: only 256 is supported", block_size);
    PKV_REQUIRE(num_blocks > 0 && num_blocks <= (INT32_MAX / kBlock), PKV_ERR_INVALID,
                "num_blocks %d out of range", num_blocks);
    pkv_allocator* a = new (std::nothrow) pkv_allocator();
    PKV_REQUIRE(a != nullptr, PKV_ERR_INVALID, "out of host memory");
    a->nblocks = num_blocks;
    a->prefix = prefix_cache != 0;
    a->nxt.assign(num_blocks, -1);
    a->prv.assign(num_blocks, -1);
    a->in_free.assign(num_blocks, 0);
    a->ref.assign(num_blocks, 0);
    a->has_hash.assign(num_blocks, 0);
    a->bhash.assign(num_blocks, 0);
    a->btok.resize(num_blocks);
    a->blk_stamp.assign(num_blocks, 0);
    a->blk_dry_ref.assign(num_blocks, 0);
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
        int32_t b = initial_order ? initial_order[i] : i;
        if (b < 0 || b >= num_blocks || seen[b]) {
            delete a;
            return fail(PKV_ERR_INVALID, "initial_order is not a permutation of 0..%d (entry %d = %d)",
                        num_blocks - 1, i, b);
        }
        seen[b] = 1;
        a->push_back(b);
    }
    *out = a;
    return PKV_OK;
}

void pkv_alloc_destroy(pkv_allocator* a) { delete a; }

int pkv_alloc_debug_constant_hash(pkv_allocator* a, int32_t enable, uint64_t value) {
    PKV_REQUIRE(a != nullptr, PKV_ERR_INVALID, "allocator is NULL");
    a->const_hash = enable != 0;
    a->const_hash_value = value;
    return PKV_OK;
}

int pkv_alloc_add_seq(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n,
                      int32_t* n_cached) {
    PKV_REQUIRE(a != nullptr && n_cached != nullptr, PKV_ERR_INVALID, "NULL argument");
    PKV_REQUIRE(n >= 0 && (n == 0 || tokens != nullptr), PKV_ERR_INVALID, "bad prompt (n=%d)", n);
    PKV_REQUIRE(a->find(seq_id) == nullptr, PKV_ERR_DUP_SEQ, "sequence %lld already admitted",
                (long long)seq_id);
    const int32_t nb = (n + kBlock - 1) / kBlock;

    // Plan every block before touching any state, so that a shortage leaves nothing changed.
    struct Step { int32_t hit; bool hashed; uint64_t h; };
    std::vector<Step> plan(nb);
    uint64_t prev = 0;
    bool hit_ok = a->prefix;
    int32_t misses = 0, hits_from_free = 0;
    for (int32_t i = 0; i < nb; ++i) {
        const int32_t* chunk = tokens + size_t(i) * kBlock;
        const bool full = int64_t(i + 1) * kBlock <= n;
        Step s{-1, false, 0};
        if (full && a->prefix) {
            s.hashed = true;
            s.h = a->hash_block(prev, chunk);
        }
        if (hit_ok && s.hashed && int64_t(i + 1) * kBlock < n) {
            auto it = a->table.find(s.h);
            if (it != a->table.end()) {
                int32_t cand = it->second;
                const std::vector<int32_t>& st = a->btok[cand];
                if (st.size() == size_t(kBlock) &&
                    std::memcmp(st.data(), chunk, sizeof(int32_t) * kBlock) == 0)
                    s.hit = cand;
            }
        }
        if (s.hit < 0) {
            hit_ok = false;
            ++misses;
        } else if (a->ref[s.hit] == 0) {
            // count each released block once, even if (under a forced collision) it is hit twice
            bool dup = false;
            for (int32_t j = 0; j < i; ++j) dup = dup || plan[j].hit == s.hit;
            if (!dup) ++hits_from_free;
        }
        plan[i] = s;
        prev = s.hashed ? s.h : 0;
    }
    if (misses > a->nfree - hits_from_free)
        return fail(PKV_ERR_NO_BLOCKS, "sequence %lld needs %d fresh blocks, %d free", (long long)seq_id,
                    misses, a->nfree - hits_from_free);

    Seq& seq = a->admit(seq_id);
    seq.blocks.reserve(nb);
    for (int32_t i = 0; i < nb; ++i) {
        const Step& s = plan[i];
        if (s.hit >= 0) {
            if (a->ref[s.hit] == 0) a->unlink(s.hit);
            ++a->ref[s.hit];
            seq.blocks.push_back(s.hit);
            seq.n_cached += kBlock;
        } else {
            int32_t b = a->pop_fresh();
            if (s.hashed) a->register_block(b, s.h, tokens + size_t(i) * kBlock);
            seq.blocks.push_back(b);
        }
        if (s.hashed) seq.last_hash = s.h;
    }
    seq.len = n;
    if (n % kBlock != 0)  // the partial last block (always fresh) keeps its tokens
        a->btok[seq.blocks.back()].assign(tokens + size_t(n / kBlock) * kBlock, tokens + n);
    *n_cached = seq.n_cached;
    return PKV_OK;
}

static int32_t append_one(pkv_allocator* a, Seq& s, int32_t token) {
    const int32_t pos = s.len;
    if (pos % kBlock == 0) s.blocks.push_back(a->pop_fresh());
    const int32_t b = s.blocks[pos / kBlock];
    a->btok[b].push_back(token);
    ++s.len;
    if (s.len % kBlock == 0 && a->prefix) {  // the block is full: register it under its chained hash
        const uint64_t h = a->hash_block(s.last_hash, a->btok[b].data());
        a->register_block(b, h, nullptr);
        s.last_hash = h;
    }
    return b * kBlock + pos % kBlock;
}

// True when the next token of s lands in a partially filled block that another sequence holds.
static bool needs_copy(const pkv_allocator* a, const Seq& s) {
    const int32_t pos = s.len;
    return pos % kBlock != 0 && a->ref[s.blocks[pos / kBlock]] > 1;
}

int pkv_alloc_append(pkv_allocator* a, int64_t seq_id, int32_t token, int32_t* slot) {
    PKV_REQUIRE(a != nullptr && slot != nullptr, PKV_ERR_INVALID, "NULL argument");
    Seq* s = a->find(seq_id);
    PKV_REQUIRE(s != nullptr, PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
    PKV_REQUIRE(s->len < INT32_MAX - 1, PKV_ERR_INVALID, "sequence too long");
    PKV_REQUIRE(!needs_copy(a, *s), PKV_ERR_INVALID,
                "sequence %lld: its last block is shared with a fork (use pkv_alloc_append_batch_cow)",
                (long long)seq_id);
    if (s->len % kBlock == 0 && a->nfree == 0)
        return fail(PKV_ERR_NO_BLOCKS, "no free block for sequence %lld", (long long)seq_id);
    *slot = append_one(a, *s, token);
    return PKV_OK;
}

int pkv_alloc_append_batch(pkv_allocator* a, const int64_t* seq_ids, const int32_t* tokens, int32_t n,
                           int32_t* slots) {
    PKV_REQUIRE(a != nullptr, PKV_ERR_INVALID, "allocator is NULL");
    PKV_REQUIRE(n >= 0, PKV_ERR_INVALID, "n = %d", n);
    if (n == 0) return PKV_OK;
    PKV_REQUIRE(seq_ids && tokens && slots, PKV_ERR_INVALID, "NULL argument");
    // Validate and count the fresh blocks the whole batch needs (a sequence may repeat).
    const uint32_t ep = a->next_epoch();
    int32_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
        Seq* s = a->find(seq_ids[i]);
        if (s == nullptr)
            return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld (batch entry %d)", (long long)seq_ids[i], i);
        PKV_REQUIRE(!needs_copy(a, *s), PKV_ERR_INVALID,
                    "sequence %lld: its last block is shared with a fork (use pkv_alloc_append_batch_cow)",
                    (long long)seq_ids[i]);
        if (s->stamp != ep) {
            s->stamp = ep;
            s->dry_len = s->len;
        }
        if (s->dry_len % kBlock == 0) ++need;
        ++s->dry_len;
    }
    if (need > a->nfree)
        return fail(PKV_ERR_NO_BLOCKS, "batch needs %d fresh blocks, %d free", need, a->nfree);
    for (int32_t i = 0; i < n; ++i) slots[i] = append_one(a, *a->find(seq_ids[i]), tokens[i]);
    return PKV_OK;
}

int pkv_alloc_fork(pkv_allocator* a, int64_t parent_id, int64_t child_id) {
    PKV_REQUIRE(a != nullptr, PKV_ERR_INVALID, "allocator is NULL");
    PKV_REQUIRE(a->find(child_id) == nullptr, PKV_ERR_DUP_SEQ, "sequence %lld exists", (long long)child_id);
    const Seq* p = a->find(parent_id);
    PKV_REQUIRE(p != nullptr, PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)parent_id);
    Seq& c = a->admit(child_id);  // slab records keep their addresses: p stays valid
    c.blocks.assign(p->blocks.begin(), p->blocks.end());  // blocks, length and hash chain
    c.len = p->len;
    c.n_cached = p->len;
    c.last_hash = p->last_hash;
    for (int32_t b : c.blocks) ++a->ref[b];
    return PKV_OK;
}

int pkv_alloc_fork_batch(pkv_allocator* a, const int64_t* parent_ids, const int64_t* child_ids, int32_t n) {
    PKV_REQUIRE(a != nullptr, PKV_ERR_INVALID, "allocator is NULL");
    PKV_REQUIRE(n >= 0, PKV_ERR_INVALID, "n = %d", n);
    if (n == 0) return PKV_OK;
    PKV_REQUIRE(parent_ids && child_ids, PKV_ERR_INVALID, "NULL argument");
    // Children sorted by id, ties by batch entry: a child listed earlier in the batch is the first
    // of its run, and a parent born in this batch is found by binary search with its entry.  The
    // checks then run in batch order, as the forks would.
    std::vector<std::pair<int64_t, int32_t>>& born = a->id_scratch;
    born.clear();
    for (int32_t i = 0; i < n; ++i) born.emplace_back(child_ids[i], i);
    std::sort(born.begin(), born.end());
    auto first_entry = [&](int64_t id) {  // the first batch entry with this child id, or n
        auto it = std::lower_bound(born.begin(), born.end(), std::make_pair(id, int32_t(-1)));
        return it != born.end() && it->first == id ? it->second : n;
    };
    for (int32_t i = 0; i < n; ++i) {
        PKV_REQUIRE(a->find(child_ids[i]) == nullptr && first_entry(child_ids[i]) == i, PKV_ERR_DUP_SEQ,
                    "sequence %lld exists (batch entry %d)", (long long)child_ids[i], i);
        PKV_REQUIRE(a->find(parent_ids[i]) != nullptr ||
                        (first_entry(parent_ids[i]) < i && parent_ids[i] != child_ids[i]),
                    PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld (batch entry %d)", (long long)parent_ids[i], i);
    }
    for (int32_t i = 0; i < n; ++i) pkv_alloc_fork(a, parent_ids[i], child_ids[i]);
    return PKV_OK;
}

int pkv_alloc_append_batch_cow(pkv_allocator* a, const int64_t* seq_ids, const int32_t* tokens, int32_t n,
                               int32_t* slots, int32_t* copy_src, int32_t* copy_dst, int32_t* copy_rows,
                               int32_t* n_copies) {
    PKV_REQUIRE(a != nullptr && n_copies != nullptr, PKV_ERR_INVALID, "NULL argument");
    PKV_REQUIRE(n >= 0, PKV_ERR_INVALID, "n = %d", n);
    *n_copies = 0;
    if (n == 0) return PKV_OK;
    PKV_REQUIRE(seq_ids && tokens && slots && copy_src && copy_dst && copy_rows, PKV_ERR_INVALID, "NULL argument");
    // Dry run on the reference counts the batch touches: fresh blocks for block starts and for copies.
    const uint32_t ep = a->next_epoch();
    int32_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
        Seq* s = a->find(seq_ids[i]);
        if (s == nullptr)
            return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld (batch entry %d)", (long long)seq_ids[i], i);
        if (s->stamp != ep) {  // (length, last block) as the batch goes
            s->stamp = ep;
            s->dry_len = s->len;
            s->dry_last = s->blocks.empty() ? -1 : s->blocks.back();
        }
        int32_t& last = s->dry_last;
        if (s->dry_len % kBlock == 0) {
            ++need;
            last = -2 - i;  // a fresh block of this batch: private
        } else if (last >= 0) {
            if (a->blk_stamp[last] != ep) {
                a->blk_stamp[last] = ep;
                a->blk_dry_ref[last] = a->ref[last];
            }
            if (a->blk_dry_ref[last] > 1) {
                ++need;
                --a->blk_dry_ref[last];
                last = -2 - i;
            }
        }
        ++s->dry_len;
    }
    if (need > a->nfree)
        return fail(PKV_ERR_NO_BLOCKS, "batch needs %d fresh blocks, %d free", need, a->nfree);
    for (int32_t i = 0; i < n; ++i) {
        Seq& s = *a->find(seq_ids[i]);
        if (needs_copy(a, s)) {
            const size_t k = size_t(s.len) / kBlock;
            const int32_t rows = s.len % kBlock;
            const int32_t src = s.blocks[k], dst = a->pop_fresh();
            --a->ref[src];
            s.blocks[k] = dst;
            const std::vector<int32_t>& st = a->btok[src];
            a->btok[dst].assign(st.begin(), st.begin() + std::min<size_t>(st.size(), size_t(rows)));
            copy_src[*n_copies] = src;
            copy_dst[*n_copies] = dst;
            copy_rows[*n_copies] = rows;
            ++*n_copies;
        }
        slots[i] = append_one(a, s, tokens[i]);
    }
    return PKV_OK;
}

int pkv_alloc_free_seq(pkv_allocator* a, int64_t seq_id) {
    PKV_REQUIRE(a != nullptr, PKV_ERR_INVALID, "allocator is NULL");
    Seq* s = a->find(seq_id);
    PKV_REQUIRE(s != nullptr, PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
    const std::vector<int32_t>& bl = s->blocks;
    for (auto r = bl.rbegin(); r != bl.rend(); ++r)
        if (--a->ref[*r] == 0) a->push_back(*r);
    a->release(seq_id);
    return PKV_OK;
}

int pkv_alloc_free_batch(pkv_allocator* a, const int64_t* seq_ids, int32_t n) {
    PKV_REQUIRE(a != nullptr, PKV_ERR_INVALID, "allocator is NULL");
    PKV_REQUIRE(n >= 0, PKV_ERR_INVALID, "n = %d", n);
    if (n == 0) return PKV_OK;
    PKV_REQUIRE(seq_ids != nullptr, PKV_ERR_INVALID, "NULL argument");
    const uint32_t ep = a->next_epoch();
    for (int32_t i = 0; i < n; ++i) {
        Seq* s = a->find(seq_ids[i]);
        const bool fresh = s != nullptr && s->stamp != ep;  // known, and not listed twice
        PKV_REQUIRE(fresh, PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld (batch entry %d)", (long long)seq_ids[i], i);
        s->stamp = ep;
    }
    for (int32_t i = 0; i < n; ++i) pkv_alloc_free_seq(a, seq_ids[i]);
    return PKV_OK;
}

int pkv_alloc_num_free(const pkv_allocator* a, int32_t* out) {
    PKV_REQUIRE(a != nullptr && out != nullptr, PKV_ERR_INVALID, "NULL argument");
    *out = a->nfree;
    return PKV_OK;
}

int pkv_alloc_block_tables(const pkv_allocator* a, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                           int32_t* out, int32_t* context_lens) {
    PKV_REQUIRE(a != nullptr, PKV_ERR_INVALID, "allocator is NULL");
    PKV_REQUIRE(n >= 0 && max_blocks >= 0, PKV_ERR_INVALID, "n = %d, max_blocks = %d", n, max_blocks);
    if (n == 0) return PKV_OK;
    PKV_REQUIRE(seq_ids != nullptr && (out != nullptr || max_blocks == 0), PKV_ERR_INVALID, "NULL argument");
    for (int32_t i = 0; i < n; ++i) {
        const Seq* s = a->find(seq_ids[i]);
        if (s == nullptr) return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
        if (s->blocks.size() > size_t(max_blocks))
            return fail(PKV_ERR_SMALL_BUFFER, "sequence %lld holds %zu blocks > max_blocks %d",
                        (long long)seq_ids[i], s->blocks.size(), max_blocks);
    }
    for (int32_t i = 0; i < n; ++i) {
        const Seq& s = *a->find(seq_ids[i]);
        int32_t* row = out + size_t(i) * max_blocks;
        const size_t nb = s.blocks.size();
        std::copy(s.blocks.begin(), s.blocks.end(), row);
        std::fill(row + nb, row + max_blocks, -1);
        if (context_lens) context_lens[i] = s.len;
    }
    return PKV_OK;
}

int pkv_alloc_prefill_slots(const pkv_allocator* a, const int64_t* seq_ids, int32_t n, int32_t* cu_seqlens_q,
                            int32_t* seqlens_k, int32_t* slot_mapping, int32_t cap, int32_t* n_slots) {
    PKV_REQUIRE(a != nullptr && cu_seqlens_q != nullptr && n_slots != nullptr, PKV_ERR_INVALID, "NULL argument");
    PKV_REQUIRE(n >= 0 && cap >= 0, PKV_ERR_INVALID, "n = %d, cap = %d", n, cap);
    PKV_REQUIRE(n == 0 || (seq_ids != nullptr && seqlens_k != nullptr), PKV_ERR_INVALID, "NULL argument");
    int64_t total = 0;
    for (int32_t i = 0; i < n; ++i) {
        const Seq* s = a->find(seq_ids[i]);
        if (s == nullptr) return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
        total += int64_t(s->len) - s->n_cached;
    }
    if (total > cap) return fail(PKV_ERR_SMALL_BUFFER, "%lld new tokens > slot capacity %d", (long long)total, cap);
    PKV_REQUIRE(total == 0 || slot_mapping != nullptr, PKV_ERR_INVALID, "slot_mapping is NULL");
    int32_t k = 0;
    cu_seqlens_q[0] = 0;
    for (int32_t i = 0; i < n; ++i) {
        const Seq& s = *a->find(seq_ids[i]);
        const int32_t len = s.len;
        for (int32_t p = s.n_cached; p < len; ++p) slot_mapping[k++] = s.blocks[p / kBlock] * kBlock + p % kBlock;
        cu_seqlens_q[i + 1] = k;
        seqlens_k[i] = len;
    }
    *n_slots = k;
    return PKV_OK;
}

int pkv_alloc_prefill_segment_slots(const pkv_allocator* a, const int64_t* seq_ids, const int32_t* starts,
                                    const int32_t* ends, int32_t n, int32_t* cu_seqlens_q, int32_t* seqlens_k,
                                    int32_t* slot_mapping, int32_t cap, int32_t* n_slots) {
    PKV_REQUIRE(a != nullptr && cu_seqlens_q != nullptr && n_slots != nullptr, PKV_ERR_INVALID, "NULL argument");
    PKV_REQUIRE(n >= 0 && cap >= 0, PKV_ERR_INVALID, "n = %d, cap = %d", n, cap);
    PKV_REQUIRE(n == 0 || (seq_ids != nullptr && starts != nullptr && ends != nullptr && seqlens_k != nullptr),
                PKV_ERR_INVALID, "NULL argument");
    int64_t total = 0;
    for (int32_t i = 0; i < n; ++i) {
        const Seq* s = a->find(seq_ids[i]);
        if (s == nullptr) return fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
        const int32_t n_new = s->len - s->n_cached;
        PKV_REQUIRE(0 <= starts[i] && starts[i] <= ends[i] && ends[i] <= n_new, PKV_ERR_INVALID,
                    "segment [%d, %d) of sequence %lld with %d new tokens", starts[i], ends[i],
                    (long long)seq_ids[i], n_new);
        total += ends[i] - starts[i];
    }
    if (total > cap) return fail(PKV_ERR_SMALL_BUFFER, "%lld new tokens > slot capacity %d", (long long)total, cap);
    PKV_REQUIRE(total == 0 || slot_mapping != nullptr, PKV_ERR_INVALID, "slot_mapping is NULL");
    int32_t k = 0;
    cu_seqlens_q[0] = 0;
    for (int32_t i = 0; i < n; ++i) {
        const Seq& s = *a->find(seq_ids[i]);
        for (int32_t p = s.n_cached + starts[i]; p < s.n_cached + ends[i]; ++p)
            slot_mapping[k++] = s.blocks[p / kBlock] * kBlock + p % kBlock;
        cu_seqlens_q[i + 1] = k;
        seqlens_k[i] = s.n_cached + ends[i];
    }
    *n_slots = k;
    return PKV_OK;
}

int pkv_store_runs(const int32_t* slot_mapping, int32_t n, int32_t* runs, int32_t cap, int32_t* n_runs,
                   int32_t* max_run) {
    PKV_REQUIRE(n >= 0 && cap >= 0, PKV_ERR_INVALID, "n = %d, cap = %d", n, cap);
    PKV_REQUIRE(n_runs != nullptr && max_run != nullptr, PKV_ERR_INVALID, "NULL argument");
    PKV_REQUIRE(n == 0 || (slot_mapping != nullptr && runs != nullptr), PKV_ERR_INVALID, "NULL argument");
    int32_t r = 0, longest = 0;
    for (int32_t t = 0; t < n;) {
        const int32_t s0 = slot_mapping[t];
        if (s0 < 0) {
            ++t;
            continue;
        }
        int32_t len = 1;
        while (t + len < n && slot_mapping[t + len] == s0 + len && s0 % kBlock + len < kBlock) ++len;
        if (r >= cap) return fail(PKV_ERR_SMALL_BUFFER, "more than %d runs", cap);
        runs[2 * r] = t;
        runs[2 * r + 1] = len;
        ++r;
        longest = std::max(longest, len);
        t += len;
    }
    *n_runs = r;
    *max_run = longest;
    return PKV_OK;
}

}  // extern "C"
