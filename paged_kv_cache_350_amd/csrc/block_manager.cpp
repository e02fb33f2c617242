// Host-side page allocator (include/pa_blockmgr.h): FIFO free list, per-page
// reference counts, forks that share pages, copy-on-write on append, and the
// device-layout tables the kernels read.
// [What is PagedAttention?, "Step-by-Step Implementation Framework",
// "Copy-on-Write Memory Forking"; PagedAttention Internals, "How
// PagedAttention Works" item 2, "Copy-on-Write and Prefix Sharing",
// "Implementation: Custom Block Manager Simulation"]
//
// The free list is intrusive: doubly linked through two per-page arrays
// (every page is either in it or held by a sequence), so taking a page from
// the front, returning one to the back and pulling a cached page out of the
// middle are O(1) and never allocate.  A batch append is first dry-run to count the pages it needs --
// one per token that opens a block, one per copy-on-write -- so that running
// out of pages leaves the state untouched; the dry run's scratch lives in the
// sequences (tagged with a per-call epoch) and in per-page arrays kept
// between calls, so a decode step costs one hash lookup per sequence.
//
// Prefix caching [Paged Attention (AI terminology), "Key Points" (sharing
// row) and "Common Usage Examples" (prefix caching); PagedAttention Internals,
// "Copy-on-Write and Prefix Sharing" and "Architectural Recommendations"
// item 2]: a full page of a prompt is identified by the whole token prefix
// up to its end, since a page's K/V depends on every earlier token.  The
// identity is a 128-bit chained hash (per page, a position-salted sum of
// mixed token pairs; chained across pages through two different 64-bit
// finalizers); a lookup maps the low word to a page and checks the high
// word.  A cached page stays cached while it is held and after it returns
// to the free list; it is evicted when the free list hands it out again, so
// the least recently released cached page goes first.
#include <algorithm>
#include <stdint.h>

#include <memory>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_blockmgr.h"

struct pa_block_manager {
    int64_t num_blocks = 0;
    int32_t block_size = 0;
    // free list: head -> nxt -> ... -> tail, -1 terminated both ways
    std::vector<int32_t> nxt, prv;
    int32_t head = -1, tail = -1;
    int64_t nfree = 0;
    std::vector<int32_t> ref;      // reference count per page
    struct Seq {
        std::vector<int32_t> pages;
        int64_t len = 0;
        // scratch of the batch-append dry run, valid while epoch == the call's
        uint64_t epoch = 0;
        int64_t sim_len = 0;
        int64_t sim_opens = 0;
        bool sim_private = false;
    };
    std::unordered_map<int64_t, Seq> seqs;
    // batch-append scratch kept between calls (no per-call allocation)
    uint64_t epoch = 0;
    std::vector<int32_t> dropped;          // per page: references the dry run dropped
    std::vector<int32_t> touched;          // pages with a non-zero `dropped` entry
    std::vector<Seq*> batch;               // sequence of each token of the batch
    // prefix cache: per page its prefix key and whether it is registered
    std::vector<uint64_t> key_lo, key_hi;
    std::vector<uint8_t> cached;
    // key_lo -> page: open addressing with linear probing, at most half
    // full (one entry per cached page); built on first prompt use
    struct Slot {
        uint64_t lo;
        int32_t page;                      // -1: empty
    };
    std::vector<Slot> table;
    uint64_t mask = 0;
    std::vector<int32_t> next_hint;        // per cached page: the page last found after it
    int64_t num_cached = 0;
    std::vector<int32_t> hits;             // allocate_prompt scratch

    void unlink(int32_t page) {
        const int32_t a = prv[(size_t)page], b = nxt[(size_t)page];
        if (a >= 0) nxt[(size_t)a] = b; else head = b;
        if (b >= 0) prv[(size_t)b] = a; else tail = a;
        --nfree;
    }

    // Slot holding lo, or -1.
    int64_t find_slot(uint64_t lo) const {
        for (uint64_t i = lo & mask;; i = (i + 1) & mask) {
            if (table[(size_t)i].page < 0) return -1;
            if (table[(size_t)i].lo == lo) return (int64_t)i;
        }
    }

    // Empty slot i and shift later entries of its probe run back into the
    // hole, so no tombstones build up (deletion for linear probing, Knuth,
    // TAOCP vol. 3, section 6.4, Algorithm R).
    void erase_slot(uint64_t i) {
        for (uint64_t j = i;;) {
            j = (j + 1) & mask;
            if (table[(size_t)j].page < 0) break;
            const uint64_t home = table[(size_t)j].lo & mask;
            // move j back into i unless its home lies cyclically in (i, j]
            const bool stays = i <= j ? (i < home && home <= j) : (i < home || home <= j);
            if (!stays) {
                table[(size_t)i] = table[(size_t)j];
                i = j;
            }
        }
        table[(size_t)i].page = -1;
    }

    void uncache(int32_t page) {
        if (!cached[(size_t)page]) return;
        const int64_t at = find_slot(key_lo[(size_t)page]);
        if (at >= 0 && table[(size_t)at].page == page) erase_slot((uint64_t)at);
        cached[(size_t)page] = 0;
        --num_cached;
    }

    int32_t take() {               // caller checked nfree > 0
        const int32_t page = head;
        unlink(page);
        if (num_cached) uncache(page);   // handed out again: its old content goes
        ref[(size_t)page] = 1;
        return page;
    }

    void give_back(int32_t page) {
        prv[(size_t)page] = tail;
        nxt[(size_t)page] = -1;
        if (tail >= 0) nxt[(size_t)tail] = page; else head = page;
        tail = page;
        ++nfree;
    }

    void release(int32_t page) {
        if (--ref[(size_t)page] == 0) give_back(page);
    }

    // Page registered under (lo, hi), or -1.  `after` is the page holding
    // the prefix one page shorter (-1 at the start): its hint is tried
    // before the table, since a repeated prompt walks the same chain.
    int32_t lookup(uint64_t lo, uint64_t hi, int32_t after) const {
        if (after >= 0) {
            const int32_t h = next_hint[(size_t)after];
            if (h >= 0 && cached[(size_t)h] && key_lo[(size_t)h] == lo && key_hi[(size_t)h] == hi)
                return h;
        }
        const int64_t at = find_slot(lo);
        if (at < 0) return -1;
        const int32_t page = table[(size_t)at].page;
        return key_hi[(size_t)page] == hi ? page : -1;
    }

    // Register page under (lo, hi), replacing the page that held lo.  The
    // table has a slot for every page, so this never allocates.
    void enroll(int32_t page, uint64_t lo, uint64_t hi) {
        uint64_t i = lo & mask;
        while (table[(size_t)i].page >= 0 && table[(size_t)i].lo != lo) i = (i + 1) & mask;
        Slot& e = table[(size_t)i];
        if (e.page >= 0) {
            cached[(size_t)e.page] = 0;
            --num_cached;
        }
        e.lo = lo;
        e.page = page;
        key_lo[(size_t)page] = lo;
        key_hi[(size_t)page] = hi;
        cached[(size_t)page] = 1;
        ++num_cached;
    }

    // Build the per-page prefix-cache arrays on first use (may throw
    // bad_alloc; nothing else changes then).
    void ensure_cache() {
        if (!table.empty()) return;
        uint64_t cap = 2;
        while (cap < 2 * (uint64_t)num_blocks) cap <<= 1;
        std::vector<Slot> t((size_t)cap, Slot{0, -1});
        std::vector<uint64_t> lo((size_t)num_blocks, 0), hi((size_t)num_blocks, 0);
        std::vector<uint8_t> c((size_t)num_blocks, 0);
        std::vector<int32_t> nh((size_t)num_blocks, -1);
        table.swap(t);
        key_lo.swap(lo);
        key_hi.swap(hi);
        cached.swap(c);
        next_hint.swap(nh);
        mask = cap - 1;
    }
};

namespace {

template <typename F>
pa_status guarded(F&& f) {
    try {
        return f();
    } catch (const std::bad_alloc&) {
        return PA_ERR_HOST_MEMORY;
    } catch (...) {
        return PA_ERR_ARG;
    }
}

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

// splitmix64 output function (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014).
inline uint64_t mix_a(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

// MurmurHash3's 64-bit finalizer (Appleby, MurmurHash3, fmix64).
inline uint64_t mix_b(uint64_t z) {
    z = (z ^ (z >> 33)) * 0xff51afd7ed558ccdull;
    z = (z ^ (z >> 33)) * 0xc4ceb9fe1a85ec53ull;
    return z ^ (z >> 33);
}

// Key of the prefix that ends with `page` (bs tokens), given the key of the
// prefix before it.  Tokens are taken two at a time as one 64-bit word, and
// word j is salted with its position, so the per-page sums are
// order-sensitive; the chain makes the key depend on every earlier page.
inline void chain_key(uint64_t& lo, uint64_t& hi, const int32_t* page, int32_t bs) {
    uint64_t a = 0, b = 0;
    int32_t i = 0;
    uint64_t j = 1;
    for (; i + 1 < bs; i += 2, ++j) {
        const uint64_t w = (uint64_t)(uint32_t)page[i] | ((uint64_t)(uint32_t)page[i + 1] << 32);
        a += mix_a(w + 0x9e3779b97f4a7c15ull * j);
        b += mix_b(w ^ (0xd6e8feb86659fd93ull * j));
    }
    if (i < bs) {                                    // odd block size: last token alone
        const uint64_t w = (uint64_t)(uint32_t)page[i] | (0xffffffffull << 32);
        a += mix_a(w + 0x9e3779b97f4a7c15ull * j);
        b += mix_b(w ^ (0xd6e8feb86659fd93ull * j));
    }
    lo = mix_a(lo ^ a);
    hi = mix_b(hi + b);
}

}  // namespace

extern "C" {

pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, const int64_t* free_order,
                       pa_block_manager** out) {
    if (!out) return PA_ERR_NULL;
    *out = nullptr;
    if (num_blocks < 1 || num_blocks > ((int64_t)1 << 31) || block_size < 1) return PA_ERR_ARG;
    return guarded([&]() -> pa_status {
        pa_block_manager* bm = new pa_block_manager();
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        std::unique_ptr<pa_block_manager> hold(bm);
        const size_t nb = (size_t)num_blocks;
        bm->nxt.assign(nb, -1);
        bm->prv.assign(nb, -1);
        bm->ref.assign(nb, 0);
        bm->dropped.assign(nb, 0);
        std::vector<char> seen(free_order ? nb : 0, 0);
        for (int64_t i = 0; i < num_blocks; ++i) {
            const int64_t p = free_order ? free_order[i] : i;
            if (free_order) {
                if (p < 0 || p >= num_blocks || seen[(size_t)p]) return PA_ERR_ARG;
                seen[(size_t)p] = 1;
            }
            bm->give_back((int32_t)p);
        }
        *out = hold.release();
        return PA_OK;
    });
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int64_t pa_bm_num_free(const pa_block_manager* bm) { return bm ? bm->nfree : -1; }

int64_t pa_bm_num_seqs(const pa_block_manager* bm) { return bm ? (int64_t)bm->seqs.size() : -1; }

int64_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq_id) {
    if (!bm) return -1;
    const auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? -1 : it->second.len;
}

int64_t pa_bm_seq_pages(const pa_block_manager* bm, int64_t seq_id, int64_t cap, int32_t* pages) {
    if (!bm) return -1;
    const auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return -1;
    const std::vector<int32_t>& pg = it->second.pages;
    if (pages)
        for (int64_t i = 0; i < (int64_t)pg.size() && i < cap; ++i) pages[i] = pg[(size_t)i];
    return (int64_t)pg.size();
}

int32_t pa_bm_ref_count(const pa_block_manager* bm, int64_t page) {
    if (!bm || page < 0 || page >= bm->num_blocks) return -1;
    return bm->ref[(size_t)page];
}

int64_t pa_bm_free_list(const pa_block_manager* bm, int64_t cap, int32_t* pages) {
    if (!bm) return -1;
    if (pages) {
        int32_t p = bm->head;
        for (int64_t i = 0; p >= 0 && i < cap; ++i, p = bm->nxt[(size_t)p]) pages[i] = p;
    }
    return bm->nfree;
}

pa_status pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, int64_t num_tokens) {
    if (!bm) return PA_ERR_NULL;
    if (num_tokens < 0) return PA_ERR_ARG;
    if (bm->seqs.count(seq_id)) return PA_ERR_ARG;
    const int64_t need = blocks_for(num_tokens, bm->block_size);
    if (need > bm->nfree) return PA_ERR_OUT_OF_PAGES;
    return guarded([&]() -> pa_status {
        pa_block_manager::Seq s;
        s.pages.reserve((size_t)need);
        s.len = num_tokens;
        auto ins = bm->seqs.emplace(seq_id, std::move(s));     // may throw: nothing taken yet
        std::vector<int32_t>& pages = ins.first->second.pages;
        for (int64_t i = 0; i < need; ++i) pages.push_back(bm->take());
        return PA_OK;
    });
}

pa_status pa_bm_allocate_prompt(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                                int64_t num_tokens, int64_t* num_cached_tokens) {
    if (!bm) return PA_ERR_NULL;
    if (num_cached_tokens) *num_cached_tokens = 0;
    if (num_tokens < 0) return PA_ERR_ARG;
    if (!num_cached_tokens || (num_tokens > 0 && !tokens)) return PA_ERR_NULL;
    if (bm->seqs.count(seq_id)) return PA_ERR_ARG;
    const int32_t bs = bm->block_size;
    const int64_t total = blocks_for(num_tokens, bs);
    const int64_t full = num_tokens / bs;
    return guarded([&]() -> pa_status {
        bm->ensure_cache();
        // Walk the full pages while their prefixes are cached: those pages
        // are shared (a free one is pulled back off the free list).
        bm->hits.clear();
        bm->hits.reserve((size_t)full);
        uint64_t lo = 0x243f6a8885a308d3ull, hi = 0x13198a2e03707344ull;
        int64_t revive = 0;
        int64_t k = 0;
        int32_t prev = -1;
        for (; k < full; ++k) {
            uint64_t nlo = lo, nhi = hi;
            chain_key(nlo, nhi, tokens + k * bs, bs);
            const int32_t page = bm->lookup(nlo, nhi, prev);
            if (page < 0) break;
            bm->hits.push_back(page);
            prev = page;
            revive += bm->ref[(size_t)page] == 0;
            lo = nlo;
            hi = nhi;
        }
        if (revive + (total - k) > bm->nfree) return PA_ERR_OUT_OF_PAGES;
        pa_block_manager::Seq s;
        s.pages.reserve((size_t)total);
        s.len = num_tokens;
        auto ins = bm->seqs.emplace(seq_id, std::move(s));     // may throw: nothing changed yet
        std::vector<int32_t>& pages = ins.first->second.pages;
        for (int32_t page : bm->hits) {
            if (bm->ref[(size_t)page]++ == 0) bm->unlink(page);
            pages.push_back(page);
        }
        for (int64_t j = k; j < total; ++j) {
            const int32_t page = bm->take();
            pages.push_back(page);
            if (j < full) {                 // a full page: register its prefix
                chain_key(lo, hi, tokens + j * bs, bs);
                bm->enroll(page, lo, hi);
            }
        }
        for (int64_t j = 1; j < full; ++j)  // hints along the chain just walked
            bm->next_hint[(size_t)pages[(size_t)j - 1]] = pages[(size_t)j];
        *num_cached_tokens = k * bs;
        return PA_OK;
    });
}

int64_t pa_bm_num_cached(const pa_block_manager* bm) { return bm ? bm->num_cached : -1; }

int32_t pa_bm_page_cached(const pa_block_manager* bm, int64_t page) {
    if (!bm || page < 0 || page >= bm->num_blocks) return -1;
    return bm->cached.empty() ? 0 : bm->cached[(size_t)page];
}

pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent_id, int64_t child_id) {
    if (!bm) return PA_ERR_NULL;
    const auto it = bm->seqs.find(parent_id);
    if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
    if (bm->seqs.count(child_id)) return PA_ERR_ARG;
    return guarded([&]() -> pa_status {
        pa_block_manager::Seq child = it->second;               // copy before inserting
        bm->seqs.emplace(child_id, std::move(child));
        for (int32_t p : bm->seqs.find(child_id)->second.pages) ++bm->ref[(size_t)p];
        return PA_OK;
    });
}

pa_status pa_bm_free(pa_block_manager* bm, int64_t seq_id) {
    if (!bm) return PA_ERR_NULL;
    const auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end()) return PA_OK;
    for (int32_t p : it->second.pages) bm->release(p);
    bm->seqs.erase(it);
    return PA_OK;
}

pa_status pa_bm_append(pa_block_manager* bm, const int64_t* seq_ids, int32_t n, int64_t* slots,
                       int64_t* copies, int32_t* num_copies, int32_t max_blocks_per_seq,
                       int32_t* tables, int32_t* context_lens) {
    if (!bm) return PA_ERR_NULL;
    if (n < 0) return PA_ERR_ARG;
    if (num_copies) *num_copies = 0;
    if (n == 0) return PA_OK;
    if (!seq_ids || !slots || !copies || !num_copies) return PA_ERR_NULL;
    if (tables && (!context_lens || max_blocks_per_seq < 1)) return PA_ERR_ARG;
    const int32_t bs = bm->block_size;
    return guarded([&]() -> pa_status {
        // Dry run: the pages the batch takes, in order, without touching
        // state -- per sequence its simulated length and whether its last
        // page is already private to it in this batch, per page the
        // references dropped so far.
        const uint64_t ep = ++bm->epoch;
        bm->batch.resize((size_t)n);
        bm->touched.clear();
        int64_t need = 0;
        pa_status st = PA_OK;
        for (int32_t i = 0; i < n && st == PA_OK; ++i) {
            const auto it = bm->seqs.find(seq_ids[i]);
            if (it == bm->seqs.end()) {
                st = PA_ERR_NOT_FOUND;
                break;
            }
            pa_block_manager::Seq& q = it->second;
            bm->batch[(size_t)i] = &q;
            if (q.epoch != ep) {
                q.epoch = ep;
                q.sim_len = q.len;
                q.sim_opens = 0;
                q.sim_private = false;
            } else if (tables) {
                st = PA_ERR_ARG;            // one table row per sequence: ids must be distinct
                break;
            }
            if (q.sim_len % bs == 0) {
                ++need;                     // opens a block: fresh page
                ++q.sim_opens;
                q.sim_private = true;
            } else if (!q.sim_private) {
                const int32_t last = q.pages.back();
                if (bm->ref[(size_t)last] - bm->dropped[(size_t)last] > 1) {   // shared: copy
                    ++need;
                    if (bm->dropped[(size_t)last]++ == 0) bm->touched.push_back(last);
                }
                q.sim_private = true;
            }
            ++q.sim_len;
            if (tables && (q.sim_len + bs - 1) / bs > max_blocks_per_seq) st = PA_ERR_ARG;
        }
        for (int32_t p : bm->touched) bm->dropped[(size_t)p] = 0;
        if (st == PA_OK && need > bm->nfree) st = PA_ERR_OUT_OF_PAGES;
        if (st != PA_OK) return st;
        for (int32_t i = 0; i < n; ++i) {
            pa_block_manager::Seq& q = *bm->batch[(size_t)i];
            if (q.sim_opens) {
                q.pages.reserve(q.pages.size() + (size_t)q.sim_opens);
                q.sim_opens = 0;
            }
        }

        // Real run: nothing below allocates, so it cannot fail.
        int32_t nc = 0;
        for (int32_t i = 0; i < n; ++i) {
            pa_block_manager::Seq& q = *bm->batch[(size_t)i];
            const int64_t pos = q.len;
            int32_t* row = tables ? tables + (int64_t)i * max_blocks_per_seq : nullptr;
            if (pos % bs == 0) {
                q.pages.push_back(bm->take());
                if (row) row[q.pages.size() - 1] = q.pages.back();
            } else {
                const int32_t last = q.pages.back();
                if (bm->ref[(size_t)last] > 1) {
                    const int32_t fresh = bm->take();
                    copies[2 * (int64_t)nc] = last;
                    copies[2 * (int64_t)nc + 1] = fresh;
                    ++nc;
                    bm->release(last);
                    q.pages.back() = fresh;
                    if (row) row[q.pages.size() - 1] = fresh;
                }
            }
            q.len = pos + 1;
            if (row) context_lens[i] = (int32_t)q.len;
            slots[i] = (int64_t)q.pages.back() * bs + pos % bs;
        }
        *num_copies = nc;
        return PA_OK;
    });
}

int64_t pa_bm_shared_prefix(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n) {
    if (!bm || n < 0 || (n > 0 && !seq_ids)) return -1;
    if (n == 0) return 0;
    const auto first = bm->seqs.find(seq_ids[0]);
    if (first == bm->seqs.end()) return -1;
    const std::vector<int32_t>& p0 = first->second.pages;
    size_t pages = p0.size();
    int64_t min_len = first->second.len;
    for (int32_t i = 1; i < n; ++i) {
        const auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end()) return -1;
        const std::vector<int32_t>& pi = it->second.pages;
        size_t k = 0;
        const size_t lim = pages < pi.size() ? pages : pi.size();
        while (k < lim && pi[k] == p0[k]) ++k;
        pages = k;
        if (it->second.len < min_len) min_len = it->second.len;
    }
    const int64_t bs = bm->block_size;
    const int64_t by_pages = (int64_t)pages * bs;
    const int64_t by_len = min_len / bs * bs;
    return by_pages < by_len ? by_pages : by_len;
}

int32_t pa_bm_prefix_groups(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                            int32_t* group_start, int32_t* group_shared_len, int32_t* seq_shared_len,
                            int32_t* max_group_size, int32_t* max_shared_len) {
    if (!bm || n < 0) return -1;
    if (!group_start || (n > 0 && (!seq_ids || !group_shared_len || !seq_shared_len))) return -1;
    std::vector<int32_t> first((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        const auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end()) return -1;
        first[(size_t)i] = it->second.pages.empty() ? -1 : it->second.pages[0];
    }
    // maximal runs of consecutive sequences that start on the same page and
    // share at least one whole page; everything between two such runs is one
    // group that shares nothing (the decode reads it per sequence)
    int32_t groups = 0, max_size = 1, max_shared = 0;
    auto open_group = [&](int32_t a, int32_t e, int32_t shared) {
        group_start[groups] = a;
        group_shared_len[groups] = shared;
        for (int32_t i = a; i < e; ++i) seq_shared_len[i] = shared;
        ++groups;
        if (shared > 0) {
            max_size = std::max(max_size, e - a);
            max_shared = std::max(max_shared, shared);
        }
    };
    int32_t loose = -1;                                      // first sequence of the current sharing-nothing run
    for (int32_t a = 0; a < n;) {
        int32_t e = a + 1;
        while (e < n && first[(size_t)a] >= 0 && first[(size_t)e] == first[(size_t)a]) ++e;
        const int64_t shared = e - a >= 2 ? pa_bm_shared_prefix(bm, seq_ids + a, e - a) : 0;
        if (shared > 0) {
            if (loose >= 0) open_group(loose, a, 0);
            loose = -1;
            open_group(a, e, (int32_t)shared);
        } else if (loose < 0) {
            loose = a;
        }
        a = e;
    }
    if (loose >= 0) open_group(loose, n, 0);
    group_start[groups] = n;
    if (max_group_size) *max_group_size = max_size;
    if (max_shared_len) *max_shared_len = max_shared;
    return groups;
}

pa_status pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t n,
                             int32_t max_blocks_per_seq, int32_t pad_page, int32_t* tables,
                             int32_t* context_lens) {
    if (!bm) return PA_ERR_NULL;
    if (n < 0 || max_blocks_per_seq < 1) return PA_ERR_ARG;
    if (n == 0) return PA_OK;
    if (!seq_ids || !tables || !context_lens) return PA_ERR_NULL;
    for (int32_t i = 0; i < n; ++i) {
        const auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
        if ((int64_t)it->second.pages.size() > max_blocks_per_seq || it->second.len > INT32_MAX)
            return PA_ERR_ARG;
    }
    for (int32_t i = 0; i < n; ++i) {
        const pa_block_manager::Seq& s = bm->seqs.find(seq_ids[i])->second;
        int32_t* row = tables + (int64_t)i * max_blocks_per_seq;
        const int32_t np = (int32_t)s.pages.size();
        for (int32_t k = 0; k < np; ++k) row[k] = s.pages[(size_t)k];
        for (int32_t k = np; k < max_blocks_per_seq; ++k) row[k] = pad_page;
        context_lens[i] = (int32_t)s.len;
    }
    return PA_OK;
}

}  // extern "C"
