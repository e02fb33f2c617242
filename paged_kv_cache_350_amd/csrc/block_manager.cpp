// Host-side page allocator (include/pa_blockmgr.h): FIFO free list, per-page
// reference counts, forks that share pages, copy-on-write on append, and the
// device-layout tables the kernels read.
// [What is PagedAttention?, "Step-by-Step Implementation Framework",
// "Copy-on-Write Memory Forking"; PagedAttention Internals, "How
// PagedAttention Works" item 2, "Copy-on-Write and Prefix Sharing",
// "Implementation: Custom Block Manager Simulation"]
//
// The free list is a ring buffer of capacity num_blocks (every page is
// either in it or held by a sequence), so taking and returning pages never
// allocates.  A batch append is first dry-run to count the pages it needs --
// one per token that opens a block, one per copy-on-write -- so that running
// out of pages leaves the state untouched; the dry run's scratch lives in the
// sequences (tagged with a per-call epoch) and in per-page arrays kept
// between calls, so a decode step costs one hash lookup per sequence.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pa_blockmgr.h"

struct pa_block_manager {
    int64_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> ring;     // free list: ring[(head + i) % num_blocks], i < nfree
    int64_t head = 0;
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

    int32_t take() {               // caller checked nfree > 0
        const int32_t page = ring[(size_t)head];
        head = head + 1 == num_blocks ? 0 : head + 1;
        --nfree;
        ref[(size_t)page] = 1;
        return page;
    }

    void give_back(int32_t page) {
        int64_t tail = head + nfree;
        if (tail >= num_blocks) tail -= num_blocks;
        ring[(size_t)tail] = page;
        ++nfree;
    }

    void release(int32_t page) {
        if (--ref[(size_t)page] == 0) give_back(page);
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
        bm->ring.resize((size_t)num_blocks);
        bm->ref.assign((size_t)num_blocks, 0);
        bm->dropped.assign((size_t)num_blocks, 0);
        if (free_order) {
            std::vector<char> seen((size_t)num_blocks, 0);
            for (int64_t i = 0; i < num_blocks; ++i) {
                const int64_t p = free_order[i];
                if (p < 0 || p >= num_blocks || seen[(size_t)p]) {
                    delete bm;
                    return PA_ERR_ARG;
                }
                seen[(size_t)p] = 1;
                bm->ring[(size_t)i] = (int32_t)p;
            }
        } else {
            for (int64_t i = 0; i < num_blocks; ++i) bm->ring[(size_t)i] = (int32_t)i;
        }
        bm->nfree = num_blocks;
        *out = bm;
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
        for (int64_t i = 0; i < bm->nfree && i < cap; ++i) {
            int64_t at = bm->head + i;
            if (at >= bm->num_blocks) at -= bm->num_blocks;
            pages[i] = bm->ring[(size_t)at];
        }
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
