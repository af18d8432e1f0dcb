// Random operation sequences on the host block manager (pa_bm_*), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_block_manager_sanitized.py.  After every operation: distinct
// slots within an append, reference counts equal to the references held by the
// live sequences' tables, and free + used blocks equal to the pool size.
// Exit status 0 when every check holds.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include <set>
#include "pa.h"
int main() {
    std::mt19937_64 rng(7);
    for (int trial = 0; trial < 50; ++trial) {
        const int nb = 1 + (int)(rng() % 64);
        pa_block_manager* m = pa_bm_create(nb, 16);
        if (!m) return 1;
        std::set<long long> live;
        long long next_id = 0;
        for (int step = 0; step < 400; ++step) {
            int op = rng() % 5;
            if (op == 0) { int rc = pa_bm_add_sequence(m, next_id, rng() % 70); if (rc == PA_OK) live.insert(next_id); ++next_id; }
            else if (op == 1 && !live.empty()) { auto it = live.begin(); std::advance(it, rng() % live.size()); if (pa_bm_fork(m, *it, next_id) == PA_OK) live.insert(next_id); ++next_id; }
            else if (op == 2 && !live.empty()) { auto it = live.begin(); std::advance(it, rng() % live.size()); if (pa_bm_free(m, *it) != PA_OK) return 2; live.erase(it); }
            else if (op == 3 && !live.empty()) {
                std::vector<int64_t> ids(live.begin(), live.end());
                std::vector<int32_t> slots(ids.size()), copies(2 * ids.size());
                int32_t nc = -1;
                int rc = pa_bm_append_batch(m, ids.data(), (int32_t)ids.size(), slots.data(), copies.data(), (int32_t)ids.size(), &nc);
                if (rc != PA_OK && rc != PA_ENOMEM) return 3;
                if (rc == PA_OK) { std::set<int32_t> u(slots.begin(), slots.end()); if (u.size() != slots.size()) return 4; }
            } else if (op == 4 && !live.empty()) {
                std::vector<int64_t> ids(live.begin(), live.end());
                const int mb = 8;
                std::vector<int32_t> bt(ids.size() * mb), cl(ids.size());
                pa_bm_batch_tables(m, ids.data(), (int32_t)ids.size(), bt.data(), mb, cl.data());
            }
            // conservation: free + distinct referenced blocks == nb; refcounts == references
            std::vector<int> refs(nb, 0);
            for (long long id : live) {
                std::vector<int32_t> bt(64); int32_t cl;
                int64_t idv = id;
                if (pa_bm_batch_tables(m, &idv, 1, bt.data(), 64, &cl) != PA_OK) return 5;
                for (int j = 0; j < (cl + 15) / 16; ++j) refs[bt[j]]++;
            }
            long long used = 0;
            for (int b = 0; b < nb; ++b) { if (refs[b] != pa_bm_refcount(m, b)) return 6; if (refs[b]) ++used; }
            if (used + pa_bm_num_free(m) != nb) return 7;
        }
        pa_bm_destroy(m);
    }
    std::printf("ok\n");
    return 0;
}
