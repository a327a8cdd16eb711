// Host-side page management of the paged KV cache (declared in
// include/paged_kv_pager.h): the FIFO free list, the lazy page step of a
// decode batch, and the request pager with admission credits, lazy physical
// pages, FIFO waiting, early release and prefix sharing with copy-on-write
// ("Hours of YouTube and 85 handtyped pages of notes on LLM Inference - Start
// here", section "現在のスコープ"; "【ITニュース解説】From a Rust Inference
// Engine to Heterogeneous Serving", the paragraph on the prefix cache).
//
// Why credits alone keep the pool from running dry: a request never holds
// more pages than its credits, pages it takes are never given back before it
// ends, and each extra reference to a shared page can cause at most one
// copy.  So what the active requests may still take is at most
// (sum of their credits) - (pages live now), and admission keeps the credits
// within the pool, i.e. within (free + live) pages.
#include <algorithm>
#include <chrono>
#include <deque>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "paged_kv.h"
#include "paged_kv_pager.h"

namespace {

constexpr int kPageTokens = PKV_PAGE_TOKENS;

int64_t pages_for(int64_t tokens) { return tokens > 0 ? (tokens + kPageTokens - 1) / kPageTokens : 0; }

// FIFO of free page ids with allocation statistics; `is_free` guards against
// double frees.
class FreeList {
public:
    explicit FreeList(int64_t pool) : pool_(pool), is_free_((size_t)pool, 0) {}

    bool add_initial(int32_t page) {
        if (page < 0 || page >= pool_ || is_free_[(size_t)page]) return false;
        is_free_[(size_t)page] = 1;
        free_.push_back(page);
        return true;
    }
    void reset_peak() { peak_ = allocated(); }

    int64_t pool() const { return pool_; }
    int64_t size() const { return (int64_t)free_.size(); }
    int64_t allocated() const { return pool_ - (int64_t)free_.size(); }
    int64_t peak() const { return peak_; }

    bool pop(int32_t* page) {
        if (free_.empty()) return false;
        *page = free_.front();
        free_.pop_front();
        is_free_[(size_t)*page] = 0;
        peak_ = std::max(peak_, allocated());
        return true;
    }
    bool push(int32_t page) {
        if (page < 0 || page >= pool_ || is_free_[(size_t)page]) return false;
        is_free_[(size_t)page] = 1;
        free_.push_back(page);
        return true;
    }

private:
    int64_t pool_;
    std::deque<int32_t> free_;
    std::vector<uint8_t> is_free_;
    int64_t peak_ = 0;
};

using Clock = std::chrono::steady_clock;

struct Request {
    int32_t prompt = 0;
    int32_t allowed_new = 0;
    int64_t credits = 0;               // pages, all layers
    bool active = false;
    int32_t length = 0;                // tokens whose pages it holds
    std::vector<std::vector<int32_t>> pages;   // [layer][logical page]
    Clock::time_point submitted;

    int32_t budget_tokens() const { return prompt + allowed_new - 1; }
};

}  // namespace

struct paged_kv_free_list {
    std::mutex mu;
    FreeList fl;
    explicit paged_kv_free_list(int64_t pool) : fl(pool) {}
};

struct paged_kv_pager {
    std::mutex mu;
    FreeList fl;
    int32_t layers;
    int32_t max_context;
    std::vector<int32_t> refs;         // per page: requests holding it
    std::unordered_map<int64_t, Request> reqs;
    std::deque<int64_t> waiting;
    int64_t next_id = 1;
    int64_t credits_in_use = 0;
    int64_t live = 0;
    int64_t peak_live = 0;
    int64_t shared_refs = 0;
    int64_t copies = 0;
    int32_t active = 0, peak_active = 0, largest_batch = 0;
    int64_t submitted = 0, admitted = 0, rejected = 0, finished = 0;
    double wait_max_us = 0.0, wait_total_us = 0.0;

    paged_kv_pager(int32_t num_pages, int32_t num_layers, int32_t ctx)
        : fl(num_pages), layers(num_layers), max_context(ctx), refs((size_t)num_pages, 0) {
        for (int32_t p = 0; p < num_pages; ++p) fl.add_initial(p);
        fl.reset_peak();
    }

    int32_t take() {                    // admission guarantees a page is there
        int32_t p = -1;
        fl.pop(&p);
        refs[(size_t)p] = 1;
        ++live;
        peak_live = std::max(peak_live, live);
        return p;
    }
    void drop(int32_t p) {
        if (--refs[(size_t)p] == 0) {
            fl.push(p);
            --live;
        } else {
            --shared_refs;
        }
    }

    void write_row(const Request& r, int32_t* table, int64_t layer_stride) const {
        for (int32_t l = 0; l < layers; ++l)
            for (size_t j = 0; j < r.pages[(size_t)l].size(); ++j)
                table[(int64_t)l * layer_stride + (int64_t)j] = r.pages[(size_t)l][j];
    }

    int check_reserve(const Request* r, int32_t length, int64_t layer_stride) const {
        if (!r || !r->active) return PKV_ERR_STATE;
        if (length < 0) return PKV_ERR_INVALID_ARG;
        if (length > r->budget_tokens()) return PKV_ERR_BUDGET;
        if (layer_stride < pages_for(std::max(length, r->length))) return PKV_ERR_INVALID_ARG;
        return PKV_OK;
    }

    // New logical pages grow() would take for r, in every layer.
    int64_t fresh_pages(const Request& r, int32_t length) const {
        if (length <= r.length) return 0;
        const int64_t held = (int64_t)r.pages[0].size();
        return (pages_for(length) - std::min<int64_t>(held, pages_for(length))) * layers;
    }

    // Adds to `writers` one count per shared page (refs > 1) that the new
    // tokens of r land in.
    void shared_writes(const Request& r, int32_t length,
                       std::unordered_map<int32_t, int32_t>& writers) const {
        if (length <= r.length) return;
        const int64_t held = (int64_t)r.pages[0].size();
        for (int64_t j = r.length / kPageTokens; j < held && j * kPageTokens < length; ++j)
            for (int32_t l = 0; l < layers; ++l) {
                const int32_t p = r.pages[(size_t)l][(size_t)j];
                if (refs[(size_t)p] > 1) ++writers[p];
            }
    }

    // Copies grow() makes when the requests of one batch write into shared
    // pages: a page held by r requests and written by w of them is copied
    // min(w, r - 1) times, since the last holder left writes in place.
    int64_t copies_needed(const std::unordered_map<int32_t, int32_t>& writers) const {
        int64_t c = 0;
        for (const auto& pw : writers) c += std::min<int64_t>(pw.second, refs[(size_t)pw.first] - 1);
        return c;
    }

    // Grows r to `length` tokens (checked by check_reserve).  Pages that the
    // new tokens land in and that another request also holds are replaced
    // by private copies first.
    void grow(Request& r, int32_t length, int32_t* copy_src, int32_t* copy_dst, int32_t* nc) {
        if (length <= r.length) return;
        const int64_t held = (int64_t)r.pages[0].size();
        const int64_t first = r.length / kPageTokens;            // page of the first new token
        for (int64_t j = first; j < held && j * kPageTokens < length; ++j) {
            for (int32_t l = 0; l < layers; ++l) {
                int32_t& p = r.pages[(size_t)l][(size_t)j];
                if (refs[(size_t)p] > 1) {
                    const int32_t fresh = take();
                    if (copy_src && copy_dst) {
                        copy_src[*nc] = p;
                        copy_dst[*nc] = fresh;
                    }
                    ++*nc;
                    ++copies;
                    drop(p);
                    p = fresh;
                }
            }
        }
        const int64_t need = pages_for(length);
        for (int64_t j = held; j < need; ++j)
            for (int32_t l = 0; l < layers; ++l) r.pages[(size_t)l].push_back(take());
        r.length = length;
    }

    Request* find(int64_t id) {
        auto it = reqs.find(id);
        return it == reqs.end() ? nullptr : &it->second;
    }
};

extern "C" {

// ------------------------------------------------------------ free list --

int paged_kv_free_list_create(const int32_t* pages, int64_t num_free, int64_t pool_pages,
                              paged_kv_free_list** out) {
    if (!out || pool_pages < 1 || pool_pages > INT32_MAX || num_free < 0 || num_free > pool_pages)
        return PKV_ERR_INVALID_ARG;
    if (num_free > 0 && !pages) return PKV_ERR_INVALID_ARG;
    auto* fl = new paged_kv_free_list(pool_pages);
    for (int64_t i = 0; i < num_free; ++i) {
        if (!fl->fl.add_initial(pages[i])) {
            delete fl;
            return PKV_ERR_INVALID_ARG;
        }
    }
    fl->fl.reset_peak();
    *out = fl;
    return PKV_OK;
}

void paged_kv_free_list_destroy(paged_kv_free_list* fl) { delete fl; }

int paged_kv_free_list_pop(paged_kv_free_list* fl, int32_t* page) {
    if (!fl || !page) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(fl->mu);
    return fl->fl.pop(page) ? PKV_OK : PKV_ERR_EXHAUSTED;
}

int paged_kv_free_list_push(paged_kv_free_list* fl, int32_t page) {
    if (!fl) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(fl->mu);
    return fl->fl.push(page) ? PKV_OK : PKV_ERR_INVALID_ARG;
}

int paged_kv_free_list_stats(const paged_kv_free_list* fl, int64_t* pool_pages,
                             int64_t* peak_allocated, int64_t* free_pages) {
    if (!fl) return PKV_ERR_INVALID_ARG;
    auto* m = const_cast<paged_kv_free_list*>(fl);
    std::lock_guard<std::mutex> g(m->mu);
    if (pool_pages) *pool_pages = fl->fl.pool();
    if (peak_allocated) *peak_allocated = fl->fl.peak();
    if (free_pages) *free_pages = fl->fl.size();
    return PKV_OK;
}

int paged_kv_lazy_page_step(paged_kv_free_list* fl, int32_t* block_tables, int32_t num_layers,
                            int32_t num_seqs, int64_t bt_stride, const int32_t* context_lens,
                            int32_t* changed, int32_t* num_changed) {
    if (!fl || num_layers < 0 || num_seqs < 0 || bt_stride < 1) return PKV_ERR_INVALID_ARG;
    if (num_changed) *num_changed = 0;
    if (num_layers == 0 || num_seqs == 0) return PKV_OK;
    if (!block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(fl->mu);
    // Count first, so that an exhausted pool changes nothing.
    int64_t need = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t n = context_lens[s];
        if (n < 1) continue;
        const int64_t j = (n - 1) / kPageTokens;
        if (j >= bt_stride) return PKV_ERR_INVALID_ARG;
        for (int32_t l = 0; l < num_layers; ++l)
            if (block_tables[((int64_t)l * num_seqs + s) * bt_stride + j] < 0) ++need;
    }
    if (need > fl->fl.size()) return PKV_ERR_EXHAUSTED;
    int32_t nc = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t n = context_lens[s];
        if (n < 1) continue;
        const int64_t j = (n - 1) / kPageTokens;
        bool any = false;
        for (int32_t l = 0; l < num_layers; ++l) {
            int32_t& e = block_tables[((int64_t)l * num_seqs + s) * bt_stride + j];
            if (e < 0) {
                fl->fl.pop(&e);
                any = true;
            }
        }
        if (any) {
            if (changed) changed[nc] = s;
            ++nc;
        }
    }
    if (num_changed) *num_changed = nc;
    return PKV_OK;
}

// ---------------------------------------------------------------- pager --

int paged_kv_pager_create(int32_t num_pages, int32_t num_layers, int32_t max_context,
                          paged_kv_pager** out) {
    if (!out || num_pages < 1 || num_layers < 1 || max_context < 1) return PKV_ERR_INVALID_ARG;
    *out = new paged_kv_pager(num_pages, num_layers, max_context);
    return PKV_OK;
}

void paged_kv_pager_destroy(paged_kv_pager* pg) { delete pg; }

int paged_kv_pager_submit(paged_kv_pager* pg, int32_t prompt_tokens, int32_t max_new_tokens,
                          int64_t* request_id, int32_t* allowed_new) {
    if (!pg) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(pg->mu);
    if (prompt_tokens < 1 || prompt_tokens > pg->max_context || max_new_tokens < 1)
        return PKV_ERR_INVALID_ARG;
    Request r;
    r.prompt = prompt_tokens;
    // The last predicted token is returned without being processed, so the
    // processed prefix prompt + allowed_new - 1 must fit in the context.
    r.allowed_new = std::min(max_new_tokens, pg->max_context + 1 - prompt_tokens);
    r.credits = pages_for(r.budget_tokens()) * pg->layers;
    ++pg->submitted;
    if (r.credits > pg->fl.pool()) {
        ++pg->rejected;
        return PKV_ERR_REJECTED;
    }
    r.pages.assign((size_t)pg->layers, {});
    r.submitted = Clock::now();
    const int64_t id = pg->next_id++;
    pg->reqs.emplace(id, std::move(r));
    pg->waiting.push_back(id);
    if (request_id) *request_id = id;
    if (allowed_new) *allowed_new = pg->reqs[id].allowed_new;
    return PKV_OK;
}

int paged_kv_pager_admit(paged_kv_pager* pg, int64_t* ids, int32_t capacity,
                         int32_t* num_admitted) {
    if (!pg || capacity < 0 || (capacity > 0 && !ids)) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(pg->mu);
    int32_t n = 0;
    const auto now = Clock::now();
    while (n < capacity && !pg->waiting.empty()) {
        Request& r = pg->reqs[pg->waiting.front()];
        if (pg->credits_in_use + r.credits > pg->fl.pool()) break;   // FIFO: no overtaking
        ids[n++] = pg->waiting.front();
        pg->waiting.pop_front();
        r.active = true;
        pg->credits_in_use += r.credits;
        ++pg->active;
        ++pg->admitted;
        pg->peak_active = std::max(pg->peak_active, pg->active);
        const double us = std::chrono::duration<double, std::micro>(now - r.submitted).count();
        pg->wait_max_us = std::max(pg->wait_max_us, us);
        pg->wait_total_us += us;
    }
    if (num_admitted) *num_admitted = n;
    return PKV_OK;
}

int paged_kv_pager_reserve(paged_kv_pager* pg, int64_t request_id, int32_t length,
                           int32_t* table, int64_t layer_stride, int32_t* copy_src,
                           int32_t* copy_dst, int32_t* num_copies) {
    if (!pg || !table) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(pg->mu);
    Request* r = pg->find(request_id);
    const int st = pg->check_reserve(r, length, layer_stride);
    if (st != PKV_OK) return st;
    // Admission keeps this from failing; the check only turns a broken
    // invariant into a status instead of a bad page id.
    std::unordered_map<int32_t, int32_t> writers;
    pg->shared_writes(*r, length, writers);
    const int64_t cow = pg->copies_needed(writers);
    if (pg->fresh_pages(*r, length) + cow > pg->fl.size()) return PKV_ERR_EXHAUSTED;
    if (cow > 0 && (!copy_src || !copy_dst)) return PKV_ERR_INVALID_ARG;   // copies to report
    int32_t nc = 0;
    pg->grow(*r, length, copy_src, copy_dst, &nc);
    pg->write_row(*r, table, layer_stride);
    if (num_copies) *num_copies = nc;
    return PKV_OK;
}

int paged_kv_pager_decode_step(paged_kv_pager* pg, const int64_t* ids, const int32_t* lengths,
                               int32_t n, int32_t* tables, int64_t seq_stride,
                               int64_t layer_stride, int32_t* copy_src, int32_t* copy_dst,
                               int32_t* num_copies) {
    if (!pg || n < 0) return PKV_ERR_INVALID_ARG;
    if (num_copies) *num_copies = 0;
    if (n == 0) return PKV_OK;
    if (!ids || !lengths || !tables) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(pg->mu);
    std::vector<Request*> rs((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        rs[(size_t)i] = pg->find(ids[i]);
        const int st = pg->check_reserve(rs[(size_t)i], lengths[i], layer_stride);
        if (st != PKV_OK) return st;
        for (int32_t k = 0; k < i; ++k)
            if (ids[k] == ids[i]) return PKV_ERR_INVALID_ARG;   // one entry per request
    }
    // Count before changing anything, so that an exhausted pool changes
    // nothing.  Copies are counted per physical page over the whole batch:
    // two holders of one shared page that both write in this step make one
    // copy, not two.
    int64_t fresh = 0;
    std::unordered_map<int32_t, int32_t> writers;
    for (int32_t i = 0; i < n; ++i) {
        fresh += pg->fresh_pages(*rs[(size_t)i], lengths[i]);
        pg->shared_writes(*rs[(size_t)i], lengths[i], writers);
    }
    const int64_t cow = pg->copies_needed(writers);
    if (fresh + cow > pg->fl.size()) return PKV_ERR_EXHAUSTED;
    if (cow > 0 && (!copy_src || !copy_dst)) return PKV_ERR_INVALID_ARG;
    int32_t nc = 0;
    for (int32_t i = 0; i < n; ++i) {
        pg->grow(*rs[(size_t)i], lengths[i], copy_src, copy_dst, &nc);
        pg->write_row(*rs[(size_t)i], tables + (int64_t)i * seq_stride, layer_stride);
    }
    pg->largest_batch = std::max(pg->largest_batch, n);
    if (num_copies) *num_copies = nc;
    return PKV_OK;
}

int paged_kv_pager_share_prefix(paged_kv_pager* pg, int64_t src_id, int64_t dst_id,
                                int32_t tokens, int32_t* table, int64_t layer_stride) {
    if (!pg || !table) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(pg->mu);
    Request* src = pg->find(src_id);
    Request* dst = pg->find(dst_id);
    if (!src || !dst || src == dst || !src->active || !dst->active) return PKV_ERR_STATE;
    if (tokens < 1 || tokens > dst->prompt) return PKV_ERR_INVALID_ARG;
    if (dst->length != 0 || !dst->pages[0].empty() || src->length < tokens) return PKV_ERR_STATE;
    const int64_t np = pages_for(tokens);
    if (layer_stride < np) return PKV_ERR_INVALID_ARG;
    for (int32_t l = 0; l < pg->layers; ++l) {
        for (int64_t j = 0; j < np; ++j) {
            const int32_t p = src->pages[(size_t)l][(size_t)j];
            ++pg->refs[(size_t)p];
            ++pg->shared_refs;
            dst->pages[(size_t)l].push_back(p);
        }
    }
    dst->length = tokens;
    pg->write_row(*dst, table, layer_stride);
    return PKV_OK;
}

int paged_kv_pager_finish(paged_kv_pager* pg, int64_t request_id) {
    if (!pg) return PKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> g(pg->mu);
    auto it = pg->reqs.find(request_id);
    if (it == pg->reqs.end()) return PKV_ERR_STATE;
    Request& r = it->second;
    if (r.active) {
        for (auto& layer : r.pages)
            for (int32_t p : layer) pg->drop(p);
        pg->credits_in_use -= r.credits;
        --pg->active;
        ++pg->finished;
    } else {
        pg->waiting.erase(std::find(pg->waiting.begin(), pg->waiting.end(), request_id));
    }
    pg->reqs.erase(it);
    return PKV_OK;
}

int paged_kv_pager_get_stats(const paged_kv_pager* pg, paged_kv_pager_stats* out) {
    if (!pg || !out) return PKV_ERR_INVALID_ARG;
    auto* m = const_cast<paged_kv_pager*>(pg);
    std::lock_guard<std::mutex> g(m->mu);
    out->pool_pages = pg->fl.pool();
    out->free_pages = pg->fl.size();
    out->live_pages = pg->live;
    out->peak_live_pages = pg->peak_live;
    out->credit_pages = pg->credits_in_use;
    out->shared_refs = pg->shared_refs;
    out->copies = pg->copies;
    out->active_requests = pg->active;
    out->peak_active_requests = pg->peak_active;
    out->waiting_requests = (int32_t)pg->waiting.size();
    out->largest_decode_batch = pg->largest_batch;
    out->submitted = pg->submitted;
    out->admitted = pg->admitted;
    out->rejected = pg->rejected;
    out->finished = pg->finished;
    out->wait_max_us = pg->wait_max_us;
    out->wait_total_us = pg->wait_total_us;
    return PKV_OK;
}

}  // extern "C"
