// Randomised stress of the native page management, built with g++ and the
// address and undefined-behaviour sanitizers by tests/test_pager_asan.py (host
// code only).  Exit status 0 when every invariant held.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "paged_kv.h"
#include "paged_kv_pager.h"

#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            std::exit(1);                                          \
        }                                                          \
    } while (0)

int main(int argc, char** argv) {
    const int steps = argc > 1 ? std::atoi(argv[1]) : 20000;
    const int P = 500, L = 3, W = 40, CTX = 600;
    std::mt19937_64 rng(830);
    auto uni = [&](int lo, int hi) { return (int)std::uniform_int_distribution<int>(lo, hi)(rng); };
    paged_kv_pager* pg = nullptr;
    CHECK(paged_kv_pager_create(P, L, CTX, &pg) == PKV_OK);
    struct Req { std::vector<int32_t> table; int len = 0, budget = 0, prompt = 0; bool active = false; };
    std::map<int64_t, Req> reqs;
    std::vector<int32_t> csrc(64 * L), cdst(64 * L);
    for (int step = 0; step < steps; ++step) {
        if (uni(0, 99) < 12) {
            int64_t id; int32_t allowed;
            const int p = uni(1, CTX), n = uni(1, 400);
            const int st = paged_kv_pager_submit(pg, p, n, &id, &allowed);
            CHECK(st == PKV_OK || st == PKV_ERR_REJECTED);
            if (st == PKV_OK) {
                Req r; r.prompt = p; r.budget = p + allowed - 1; r.table.assign(L * W, -1);
                reqs[id] = r;
            }
        }
        int64_t ids[64]; int32_t na = 0;
        CHECK(paged_kv_pager_admit(pg, ids, 64, &na) == PKV_OK);
        for (int i = 0; i < na; ++i) reqs[ids[i]].active = true;
        std::vector<int64_t> act;
        for (auto& kv : reqs) if (kv.second.active) act.push_back(kv.first);
        if (!act.empty() && uni(0, 9) == 0) {
            const int64_t dst = act[(size_t)uni(0, (int)act.size() - 1)];
            const int64_t src = act[(size_t)uni(0, (int)act.size() - 1)];
            Req& d = reqs[dst]; Req& s = reqs[src];
            if (dst != src && d.len == 0 && s.len > 0) {
                const int n = std::min(s.len, d.prompt);
                CHECK(paged_kv_pager_share_prefix(pg, src, dst, n, d.table.data(), W) == PKV_OK);
                d.len = n;
            }
        }
        std::vector<int64_t> batch; std::vector<int32_t> lens; std::vector<int32_t> tabs;
        for (int64_t id : act) {
            Req& r = reqs[id];
            if (r.len < r.budget && batch.size() < 64) {
                batch.push_back(id);
                lens.push_back(std::min(r.budget, r.len + uni(1, 40)));
                tabs.insert(tabs.end(), r.table.begin(), r.table.end());
            }
        }
        if (!batch.empty()) {
            int32_t nc = 0;
            CHECK(paged_kv_pager_decode_step(pg, batch.data(), lens.data(), (int32_t)batch.size(),
                                             tabs.data(), L * W, W, csrc.data(), cdst.data(),
                                             &nc) == PKV_OK);
            for (size_t i = 0; i < batch.size(); ++i) {
                Req& r = reqs[batch[i]];
                r.table.assign(tabs.begin() + (long)(i * L * W), tabs.begin() + (long)((i + 1) * L * W));
                r.len = lens[i];
            }
            for (int i = 0; i < nc; ++i) CHECK(csrc[(size_t)i] != cdst[(size_t)i]);
        }
        for (int64_t id : act) {
            Req& r = reqs[id];
            if (r.len >= r.budget || uni(0, 49) == 0) {
                CHECK(paged_kv_pager_finish(pg, id) == PKV_OK);
                reqs.erase(id);
            }
        }
        paged_kv_pager_stats st;
        CHECK(paged_kv_pager_get_stats(pg, &st) == PKV_OK);
        CHECK(st.free_pages + st.live_pages == P);
        CHECK(st.live_pages <= st.credit_pages);
        std::map<int32_t, int> refs;
        for (auto& kv : reqs) {
            if (!kv.second.active) continue;
            const int held = (kv.second.len + 15) / 16;
            for (int l = 0; l < L; ++l)
                for (int j = 0; j < held; ++j) {
                    const int32_t p = kv.second.table[(size_t)(l * W + j)];
                    CHECK(p >= 0 && p < P);
                    ++refs[p];
                }
        }
        long extra = 0;
        for (auto& kv : refs) extra += kv.second - 1;
        CHECK((long)refs.size() == st.live_pages && extra == st.shared_refs);
    }
    paged_kv_pager_stats st;
    paged_kv_pager_get_stats(pg, &st);
    for (auto& kv : reqs) CHECK(paged_kv_pager_finish(pg, kv.first) == PKV_OK);
    paged_kv_pager_stats end;
    paged_kv_pager_get_stats(pg, &end);
    CHECK(end.free_pages == P && end.live_pages == 0 && end.credit_pages == 0);
    paged_kv_pager_destroy(pg);
    std::printf("ok: %lld admitted, %lld copies, peak %lld live pages\n", (long long)st.admitted,
                (long long)st.copies, (long long)st.peak_live_pages);
    return 0;
}
