// Seeded random operation sequences against the host block manager's C ABI, built with the address
// and undefined-behaviour sanitizers by tests/test_alloc_sanitizers.py (CPU only).
//
// Every entry point of the block manager runs many times, error paths included (unknown and repeated
// ids, pool exhaustion, appends into shared partial blocks, forced hash collisions).  After every
// operation the driver checks what the ABI exposes:
//   * the blocks referenced by live sequences are exactly num_blocks - num_free distinct ids;
//   * every table row holds ceil(len / 256) valid ids, distinct within the row, padded with -1;
//   * each sequence has the length the driver expects;
//   * a failed call leaves num_free and every table unchanged.
// Exit status 0 means every check passed (the sanitizers abort on the first memory or UB error).
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pkv.h"

namespace {

constexpr int kBlock = PKV_BLOCK_SIZE;
int g_checks = 0;
int g_copies = 0, g_no_blocks = 0, g_refused = 0;  // coverage of the interesting paths

#define CHECK(cond, ...)                                                 \
    do {                                                                 \
        ++g_checks;                                                      \
        if (!(cond)) {                                                   \
            std::fprintf(stderr, "check failed at line %d: ", __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                           \
            std::fprintf(stderr, " (%s)\n", pkv_last_error());           \
            std::exit(1);                                                \
        }                                                                \
    } while (0)

struct Model {
    pkv_allocator* a = nullptr;
    int32_t nb = 0;
    std::map<int64_t, int32_t> len;  // live sequence -> expected length
};

std::vector<int32_t> tables(const Model& m, const std::vector<int64_t>& ids, int32_t width,
                            std::vector<int32_t>* lens = nullptr) {
    std::vector<int32_t> out(ids.size() * size_t(width) + 1), l(ids.size() + 1);
    const int rc = pkv_alloc_block_tables(m.a, ids.data(), int32_t(ids.size()), width, out.data(), l.data());
    CHECK(rc == PKV_OK, "block_tables rc %d", rc);
    if (lens) *lens = l;
    return out;
}

void check_state(const Model& m) {
    std::vector<int64_t> ids;
    for (auto& kv : m.len) ids.push_back(kv.first);
    int32_t width = 1;
    for (auto& kv : m.len) width = std::max(width, (kv.second + kBlock - 1) / kBlock);
    std::vector<int32_t> lens;
    const std::vector<int32_t> t = tables(m, ids, width, &lens);
    std::set<int32_t> used;
    for (size_t i = 0; i < ids.size(); ++i) {
        const int32_t L = m.len.at(ids[i]);
        CHECK(lens[i] == L, "sequence %lld length %d, expected %d", (long long)ids[i], lens[i], L);
        std::set<int32_t> row;
        const int32_t nblk = (L + kBlock - 1) / kBlock;
        for (int32_t j = 0; j < width; ++j) {
            const int32_t b = t[i * width + j];
            if (j < nblk) {
                CHECK(b >= 0 && b < m.nb, "block id %d out of range", b);
                CHECK(row.insert(b).second, "block %d twice in one table row", b);
                used.insert(b);
            } else {
                CHECK(b == -1, "padding %d", b);
            }
        }
    }
    int32_t nfree = -1;
    CHECK(pkv_alloc_num_free(m.a, &nfree) == PKV_OK, "num_free");
    CHECK(int32_t(used.size()) == m.nb - nfree, "%zu blocks in use, %d free of %d", used.size(), nfree, m.nb);
}

// Snapshot used to check that a failing call changed nothing.
struct Snap {
    int32_t nfree;
    std::vector<int32_t> tab;
};
Snap snap(const Model& m) {
    Snap s;
    pkv_alloc_num_free(m.a, &s.nfree);
    std::vector<int64_t> ids;
    for (auto& kv : m.len) ids.push_back(kv.first);
    s.tab = ids.empty() ? std::vector<int32_t>() : tables(m, ids, 64);
    return s;
}
void same(const Model& m, const Snap& s, const char* what) {
    const Snap t = snap(m);
    CHECK(t.nfree == s.nfree && t.tab == s.tab, "failed %s changed the state", what);
}

}  // namespace

int main(int argc, char** argv) {
    const int seeds = argc > 1 ? std::atoi(argv[1]) : 6;
    const int ops = argc > 2 ? std::atoi(argv[2]) : 1500;
    for (int seed = 0; seed < seeds; ++seed) {
        std::mt19937_64 rng(uint64_t(seed) * 7919 + 1);
        auto pick = [&](int lo, int hi) { return lo + int(rng() % uint64_t(hi - lo + 1)); };
        Model m;
        m.nb = pick(24, 64);
        std::vector<int32_t> order(m.nb);
        for (int i = 0; i < m.nb; ++i) order[i] = i;
        std::shuffle(order.begin(), order.end(), rng);
        CHECK(pkv_alloc_create(m.nb, kBlock, order.data(), seed % 3 != 2, &m.a) == PKV_OK, "create");
        if (seed % 4 == 3) pkv_alloc_debug_constant_hash(m.a, 1, 42);  // every block collides
        std::vector<int32_t> shared(700);
        for (auto& x : shared) x = pick(0, 40);
        int64_t next = 0;
        auto live = [&]() {
            std::vector<int64_t> v;
            for (auto& kv : m.len) v.push_back(kv.first);
            return v;
        };
        auto any_live = [&]() { auto v = live(); return v[rng() % v.size()]; };
        for (int op = 0; op < ops; ++op) {
            const int kind = pick(0, 11);
            if (kind <= 1 || m.len.empty()) {  // admit a prompt, often sharing a prefix
                const int n = pick(0, 900), share = std::min(n, pick(0, 2) * 256 + pick(0, 1) * 150);
                std::vector<int32_t> toks(shared.begin(), shared.begin() + share);
                while (int(toks.size()) < n) toks.push_back(pick(0, 1 << 20));
                const Snap s = snap(m);
                int32_t cached = -1;
                const int rc = pkv_alloc_add_seq(m.a, next, toks.data(), n, &cached);
                if (rc == PKV_OK) {
                    CHECK(cached >= 0 && cached <= n && cached % kBlock == 0, "n_cached %d of %d", cached, n);
                    m.len[next] = n;
                } else {
                    CHECK(rc == PKV_ERR_NO_BLOCKS, "add_seq rc %d", rc);
                    ++g_no_blocks;
                    same(m, s, "add_seq");
                }
                ++next;
            } else if (kind == 2) {  // single append (refused on a shared partial block)
                const int64_t id = any_live();
                const Snap s = snap(m);
                int32_t slot = -1;
                const int rc = pkv_alloc_append(m.a, id, pick(0, 9), &slot);
                if (rc == PKV_OK) {
                    CHECK(slot >= 0 && slot < m.nb * kBlock && slot % kBlock == m.len[id] % kBlock, "slot %d", slot);
                    ++m.len[id];
                } else {
                    CHECK(rc == PKV_ERR_NO_BLOCKS || rc == PKV_ERR_INVALID, "append rc %d", rc);
                    (rc == PKV_ERR_INVALID ? g_refused : g_no_blocks) += 1;
                    same(m, s, "append");
                }
            } else if (kind <= 4) {  // copy-on-write batch append
                std::vector<int64_t> ids;
                const int k = pick(1, 8);
                for (int i = 0; i < k; ++i) ids.push_back(any_live());
                std::vector<int32_t> toks(k), slots(k), src(k), dst(k), rows(k);
                for (auto& x : toks) x = pick(0, 9);
                const Snap s = snap(m);
                int32_t nc = -1;
                const int rc = pkv_alloc_append_batch_cow(m.a, ids.data(), toks.data(), k, slots.data(), src.data(),
                                                         dst.data(), rows.data(), &nc);
                if (rc == PKV_OK) {
                    CHECK(nc >= 0 && nc <= k, "n_copies %d", nc);
                    g_copies += nc;
                    for (int i = 0; i < nc; ++i)
                        CHECK(src[i] >= 0 && src[i] < m.nb && dst[i] >= 0 && dst[i] < m.nb && src[i] != dst[i] &&
                                  rows[i] > 0 && rows[i] < kBlock, "copy %d -> %d, %d rows", src[i], dst[i], rows[i]);
                    for (int i = 0; i < k; ++i) {
                        CHECK(slots[i] >= 0 && slots[i] < m.nb * kBlock && slots[i] % kBlock == m.len[ids[i]] % kBlock,
                              "slot %d", slots[i]);
                        ++m.len[ids[i]];
                    }
                } else {
                    CHECK(rc == PKV_ERR_NO_BLOCKS, "append_batch_cow rc %d", rc);
                    same(m, s, "append_batch_cow");
                }
            } else if (kind == 5) {  // plain batch append
                std::vector<int64_t> ids;
                const int k = pick(1, 5);
                for (int i = 0; i < k; ++i) ids.push_back(any_live());
                std::vector<int32_t> toks(k, 1), slots(k);
                const Snap s = snap(m);
                const int rc = pkv_alloc_append_batch(m.a, ids.data(), toks.data(), k, slots.data());
                if (rc == PKV_OK) {
                    for (int i = 0; i < k; ++i) ++m.len[ids[i]];
                } else {
                    CHECK(rc == PKV_ERR_NO_BLOCKS || rc == PKV_ERR_INVALID, "append_batch rc %d", rc);
                    same(m, s, "append_batch");
                }
            } else if (kind <= 7) {  // forks, single or batched (a child may fork again)
                const int k = pick(1, 4);
                std::vector<int64_t> par, chi;
                for (int i = 0; i < k; ++i) {
                    par.push_back(i > 0 && pick(0, 1) ? chi.back() : any_live());
                    chi.push_back(next++);
                }
                const Snap s = snap(m);
                const int rc = k == 1 ? pkv_alloc_fork(m.a, par[0], chi[0])
                                      : pkv_alloc_fork_batch(m.a, par.data(), chi.data(), k);
                CHECK(rc == PKV_OK, "fork rc %d", rc);
                for (int i = 0; i < k; ++i) m.len[chi[i]] = m.len.at(par[i]);
                (void)s;
            } else if (kind == 8) {  // error paths: unknown ids, repeated ids
                const Snap s = snap(m);
                int32_t slot;
                CHECK(pkv_alloc_append(m.a, next + 1000, 1, &slot) == PKV_ERR_UNKNOWN_SEQ, "unknown append");
                const int64_t id = any_live();
                CHECK(pkv_alloc_fork(m.a, id, id) == PKV_ERR_DUP_SEQ, "fork onto itself");
                const int64_t two[2] = {id, id};
                CHECK(pkv_alloc_free_batch(m.a, two, 2) == PKV_ERR_UNKNOWN_SEQ, "repeated free");
                const int64_t pc[2] = {next + 5, next + 6};
                CHECK(pkv_alloc_fork_batch(m.a, pc, pc + 1, 1) == PKV_ERR_UNKNOWN_SEQ, "fork of unknown");
                same(m, s, "error paths");
            } else if (kind == 9) {  // metadata calls
                auto ids = live();
                int32_t total = 0;
                for (auto id : ids) total += m.len[id];
                std::vector<int32_t> cu(ids.size() + 1), lk(ids.size()), sl(size_t(total) + 1);
                int32_t n_slots = -1;
                CHECK(pkv_alloc_prefill_slots(m.a, ids.data(), int32_t(ids.size()), cu.data(), lk.data(), sl.data(),
                                              total, &n_slots) == PKV_OK, "prefill_slots");
                CHECK(n_slots >= 0 && n_slots <= total && cu.back() == n_slots, "n_slots %d", n_slots);
                std::vector<int32_t> runs(2 * size_t(n_slots) + 2);
                int32_t nr = -1, mx = -1;
                CHECK(pkv_store_runs(sl.data(), n_slots, runs.data(), n_slots, &nr, &mx) == PKV_OK, "store_runs");
                int32_t covered = 0;
                for (int i = 0; i < nr; ++i) covered += runs[2 * i + 1];
                CHECK(covered == n_slots && mx <= kBlock, "runs cover %d of %d", covered, n_slots);
            } else {  // end sequences, one or several
                auto ids = live();
                std::shuffle(ids.begin(), ids.end(), rng);
                const int k = std::min<int>(int(ids.size()), pick(1, 3));
                const int rc = k == 1 ? pkv_alloc_free_seq(m.a, ids[0]) : pkv_alloc_free_batch(m.a, ids.data(), k);
                CHECK(rc == PKV_OK, "free rc %d", rc);
                for (int i = 0; i < k; ++i) m.len.erase(ids[i]);
            }
            check_state(m);
        }
        pkv_alloc_destroy(m.a);
    }
    std::printf("alloc_stress: %d seeds x %d operations, %d checks passed (%d block copies, %d pool "
                "exhaustions, %d refused appends)\n", seeds, ops, g_checks, g_copies, g_no_blocks, g_refused);
    // the sequences must have reached every path the checks are for
    return g_copies > 0 && g_no_blocks > 0 && g_refused > 0 ? 0 : 2;
}
