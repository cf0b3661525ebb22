// Sanitizer driver for the host side of libseedmm (test infrastructure): argument
// validation of every entry point, the size functions, and the expert cache planner, all
// of which run on the host without touching a GPU.  Built with AddressSanitizer and
// UBSan on the host code; exit status 0 = clean.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/seedmm.h"

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static uint64_t rng = 0xC0FFEEu;
static uint32_t next32() {
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (uint32_t)((rng * 2685821657736338717ull) >> 32);
}

int main() {
    void* F = (void*)(uintptr_t)0x100000;   // aligned, never dereferenced (validation fails first)
    seedmm_mat m = {(const uint16_t*)F, (const uint16_t*)F, (const uint8_t*)F, (const int32_t*)F};
    // sizes
    CHECK(seedmm_moe_workspace_bytes(64, 8, 100, 2048, 1024) > 0);
    CHECK(seedmm_moe_workspace_bytes(-1, 8, 100, 2048, 1024) == 0);
    CHECK(seedmm_search_table_bytes(4) > seedmm_search_table_bytes(3));
    CHECK(seedmm_search_table_bytes(2) == 0);
    size_t off[9];
    CHECK(seedmm_cache_record_layout(2048, 1024, 4, off) % 256 == 0);
    CHECK(seedmm_cache_record_layout(2048, 1024, 5, off) == 0);
    // argument errors: each returns before any HIP call
    CHECK(seedmm_gemv((const uint16_t*)F, (const uint16_t*)F, (const uint8_t*)F, 0, (const float*)F, (float*)F, 16, 12, 4) == SEEDMM_EINVAL);
    CHECK(seedmm_gemv_ex(nullptr, nullptr, nullptr, 0, F, 1, 16, (float*)F, 16, 16, 16, 4, 1, nullptr) == SEEDMM_EINVAL);
    CHECK(seedmm_reconstruct((const uint16_t*)F, (const uint16_t*)F, (const uint8_t*)F, 0, (char*)F + 2, 0, 16, 16, 4, nullptr) == SEEDMM_EALIGN);
    CHECK(seedmm_moe_dispatch((const int32_t*)F, 4, 0, 8, (int32_t*)F, (int32_t*)F, nullptr) == SEEDMM_EINVAL);
    CHECK(seedmm_moe((const int32_t*)F, (const float*)F, 4, 9, F, (float*)F, 8, 64, 32, 4, m, m, m, F, 1 << 20, nullptr) == SEEDMM_EINVAL);
    CHECK(seedmm_moe((const int32_t*)F, (const float*)F, 4, 2, F, (float*)F, 8, 64, 32, 4, m, m, m, F, 16, nullptr) == SEEDMM_EWORKSPACE);
    seedmm_side side = {F, nullptr, F};
    CHECK(seedmm_moe_ex((const int32_t*)F, (const float*)F, 4, 2, F, (float*)F, 8, 64, 64, 4, nullptr, m, m, m, F, 1 << 20, (char*)F + 4096, &side) == SEEDMM_EINVAL);
    CHECK(seedmm_moe_ex((const int32_t*)F, (const float*)F, 4, 2, F, (float*)F, 8, 64, 64, 0, nullptr, m, m, m, F, 1 << 20, nullptr, nullptr) == SEEDMM_EINVAL);
    CHECK(seedmm_moe_noalloc((const int32_t*)F, (const float*)F, 128, 8, F, (float*)F, 100, 2048, 1024, 4, m, m, m, nullptr) == SEEDMM_ESCRATCH);
    CHECK(seedmm_moe_mixed((const int32_t*)F, (const float*)F, 4, 2, F, (float*)F, 8, 64, 64, nullptr, m, m, m, F, 1 << 20, nullptr) == SEEDMM_EINVAL);
    CHECK(seedmm_search((const float*)F, 16, nullptr, 4, 16, 4, -4, (uint16_t*)F, (uint16_t*)F, (uint8_t*)F, nullptr, nullptr, nullptr) == SEEDMM_EINVAL);
    CHECK(seedmm_search_prepare(4, (char*)F + 16, seedmm_search_table_bytes(4), nullptr) == SEEDMM_EALIGN);
    for (int st = -8; st <= 2; ++st) CHECK(seedmm_strerror(st) != nullptr);
    // expert cache planner: random call sequences against a simple model of its rules
    for (int trial = 0; trial < 40; ++trial) {
        const int E = 4 + (int)(next32() % 60), S = 1 + (int)(next32() % E), k = 1 + (int)(next32() % (S < 8 ? S : 8));
        const int H = 64, I = 32, P = 3 + (int)(next32() % 2);
        const size_t nstate = seedmm_cache_state_bytes(E, S), ndev = seedmm_cache_device_bytes(E, H, I, P, S);
        CHECK(nstate > 0 && ndev > 0);
        std::vector<uint64_t> state((nstate + 7) / 8);
        CHECK(seedmm_cache_init(state.data(), nstate, E, H, I, P, S, F, (const int32_t*)F, F, ndev) == SEEDMM_OK);
        seedmm_cache* c = (seedmm_cache*)state.data();
        CHECK(seedmm_cache_init(state.data(), nstate - 1, E, H, I, P, S, F, (const int32_t*)F, F, ndev) == SEEDMM_EINVAL);
        CHECK(seedmm_cache_init(state.data(), nstate, E, H, I, P, S, F, (const int32_t*)F, F, ndev) == SEEDMM_OK);
        std::vector<int32_t> slot_of(E, -1);
        std::vector<int32_t> loads(2 * S);
        uint64_t misses = 0;
        for (int call = 0; call < 50; ++call) {
            const int T = 1 + (int)(next32() % 3);
            std::vector<int32_t> ids(T * k);
            for (int t = 0; t < T; ++t)
                for (int s = 0; s < k; ++s) {
                    int e;
                    bool dup;
                    do {   // distinct within a token
                        e = (int)(next32() % E);
                        dup = false;
                        for (int q = 0; q < s; ++q) dup = dup || ids[t * k + q] == e;
                    } while (dup);
                    ids[t * k + s] = e;
                }
            int nl = -1;
            const int rc = seedmm_cache_plan(c, ids.data(), T, k, loads.data(), &nl);
            std::vector<int> distinct;
            for (int v : ids) {
                bool seen = false;
                for (int d : distinct) seen = seen || d == v;
                if (!seen) distinct.push_back(v);
            }
            if ((int)distinct.size() > S) {
                CHECK(rc == SEEDMM_ECAPACITY);
                continue;
            }
            CHECK(rc == SEEDMM_OK && nl >= 0 && nl <= S);
            misses += (uint64_t)nl;
            for (int i = 0; i < nl; ++i) {
                const int e = loads[2 * i], sl = loads[2 * i + 1];
                CHECK(e >= 0 && e < E && sl >= 0 && sl < S);
                for (int q = 0; q < E; ++q)
                    if (slot_of[q] == sl) slot_of[q] = -1;   // the slot's old expert leaves
                slot_of[e] = sl;
            }
            for (int d : distinct) CHECK(slot_of[d] >= 0);   // every used expert resident
        }
        int32_t bad[2] = {E, 0};
        int nl;
        CHECK(seedmm_cache_plan(c, bad, 1, 2, loads.data(), &nl) == SEEDMM_EINVAL);
        uint64_t st[5];
        CHECK(seedmm_cache_stats(c, st) == SEEDMM_OK && st[3] == misses && st[2] + st[3] == st[1]);
        CHECK(seedmm_cache_reset(c) == SEEDMM_OK);
        CHECK(seedmm_cache_stats(c, st) == SEEDMM_OK && st[0] == 0);
    }
    printf("host sanitizer driver: clean\n");
    return 0;
}
