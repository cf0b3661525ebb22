// Expert cache: a layer's routed experts stay in pinned host memory and the recently used
// ones sit in S device slots (NanoSeedLM README, "Highlights" and "With the engine";
// eviction by least recent use, documentation index "Results").
//
// Each expert is one record of its nine streams (gate, up, down x seeds, coefs, codes),
// laid out identically in the host pack and in a device slot, so loading an expert is one
// host-to-device copy (SDMA) of the record.  The host decides: each call plans on the
// host copy of the routing which experts to load and where, enqueues their record copies
// on the caller's stream, updates the device expert -> slot map with one small kernel
// whose changes travel as launch arguments (no staging buffer, nothing to wait for), and
// runs the layer kernels with the map.  Stream order makes the copies wait for the
// previous call's kernels, so a slot is never overwritten while it is read.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/seedmm.h"
#include "moe_layer.hpp"

namespace {

constexpr uint64_t kMagic = 0x5eedcace0002ull;
constexpr int kMaxE = 4096;

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }
size_t up8(size_t v) { return (v + 7) & ~(size_t)7; }

bool shape_ok(int H, int I, int P) {
    if (P != 3 && P != 4) return false;
    if (H <= 0 || I <= 0 || H % 8 != 0 || I % 8 != 0) return false;
    const int64_t n = (int64_t)I * (H / 8);
    return (n * P) % 4 == 0 && n % 2 == 0;
}

bool counts_ok(int E, int S) { return E >= 1 && E <= kMaxE && S >= 1 && S <= E; }

// Offsets of the nine parts of an expert record, and the record size.
size_t record_layout(int H, int I, int P, size_t off[9]) {
    const int64_t n = (int64_t)I * (H / 8);
    const size_t part[3] = {(size_t)n * 2, (size_t)(n * P / 4) * 2, (size_t)(n / 2)};
    size_t o = 0;
    for (int m = 0; m < 3; ++m)
        for (int k = 0; k < 3; ++k) {
            off[3 * m + k] = o;
            o = up256(o + part[k]);
        }
    return o;
}

}  // namespace

// The cache state, placed in the caller's host buffer; the tables follow it.
struct seedmm_cache {
    uint64_t magic;
    int E, H, I, P, S;
    size_t record;             // bytes of one expert record
    size_t stream_bytes;       // bytes of the nine streams of one expert (without padding)
    const char* host_pack;     // pinned host, E records
    char* slots_dev;           // device, S records
    seedmm_mat slot0[3];       // gate, up, down streams of slot 0 (+ device exp_bias [E])
    int32_t* slot_map_dev;     // device int32[E]
    bool device_map_valid;     // the device map holds every resident expert's slot
    uint64_t step;
    uint64_t stats[5];
    int32_t* slot_of;          // [E]: slot of expert e, or -1
    int32_t* expert_of;        // [S]: expert in slot s, or -1
    uint64_t* last_use;        // [S]: step of the slot's last use
    uint8_t* used;             // [E]: scratch of one plan
    int32_t* loads;            // [2*S]: scratch of one call
};

namespace {

size_t state_bytes(int E, int S) {
    return up8(sizeof(seedmm_cache)) + up8((size_t)E * 4) + up8((size_t)S * 4) +
           (size_t)S * 8 + up8((size_t)E) + up8((size_t)S * 8);
}

size_t device_bytes(int E, int H, int I, int P, int S) {
    size_t off[9];
    return up256(record_layout(H, I, P, off) * (size_t)S) + up256((size_t)E * 4);
}

void clear_tables(seedmm_cache* c) {
    for (int e = 0; e < c->E; ++e) c->slot_of[e] = -1;
    for (int s = 0; s < c->S; ++s) {
        c->expert_of[s] = -1;
        c->last_use[s] = 0;
    }
    c->device_map_valid = false;
}

bool valid(const seedmm_cache* c) { return c && c->magic == kMagic; }

// Changes to the device map, carried as launch arguments.
constexpr int kUpd = 240;
struct MapUpdate {
    int n;
    int32_t idx[kUpd];
    int32_t val[kUpd];
};

__global__ __launch_bounds__(256) void k_map_update(int32_t* map, const MapUpdate u) {
    const int t = threadIdx.x;
    if (t < u.n) map[u.idx[t]] = u.val[t];
}

__global__ __launch_bounds__(256) void k_map_fill(int32_t* map, int n, int32_t v) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) map[i] = v;
}

}  // namespace

extern "C" {

size_t seedmm_cache_record_layout(int H, int I, int P, size_t offsets[9]) {
    if (!shape_ok(H, I, P)) return 0;
    size_t off[9];
    const size_t r = record_layout(H, I, P, off);
    if (offsets)
        for (int i = 0; i < 9; ++i) offsets[i] = off[i];
    return r;
}

size_t seedmm_cache_state_bytes(int E, int S) {
    if (!counts_ok(E, S)) return 0;
    return state_bytes(E, S);
}

size_t seedmm_cache_device_bytes(int E, int H, int I, int P, int S) {
    if (!counts_ok(E, S) || !shape_ok(H, I, P)) return 0;
    return device_bytes(E, H, I, P, S);
}

int seedmm_cache_init(void* state, size_t state_bytes_given, int E, int H, int I, int P, int S,
                      const void* host_pack, const int32_t* exp_bias, void* device,
                      size_t device_bytes_given) {
    if (!state || !device || !host_pack || !exp_bias) return SEEDMM_EINVAL;
    if (!counts_ok(E, S) || !shape_ok(H, I, P)) return SEEDMM_EINVAL;
    if (((uintptr_t)state & 7) != 0 || ((uintptr_t)device & 255) != 0) return SEEDMM_EALIGN;
    if (state_bytes_given < state_bytes(E, S)) return SEEDMM_EINVAL;
    if (device_bytes_given < device_bytes(E, H, I, P, S)) return SEEDMM_EINVAL;

    seedmm_cache* c = (seedmm_cache*)state;
    memset(c, 0, sizeof(*c));
    c->E = E; c->H = H; c->I = I; c->P = P; c->S = S;
    size_t off[9];
    c->record = record_layout(H, I, P, off);
    const int64_t n = (int64_t)I * (H / 8);
    c->stream_bytes = 3 * ((size_t)n * 2 + (size_t)(n * P / 4) * 2 + (size_t)(n / 2));
    char* t = (char*)state + up8(sizeof(seedmm_cache));
    c->slot_of = (int32_t*)t;   t += up8((size_t)E * 4);
    c->expert_of = (int32_t*)t; t += up8((size_t)S * 4);
    c->last_use = (uint64_t*)t; t += (size_t)S * 8;
    c->used = (uint8_t*)t;      t += up8((size_t)E);
    c->loads = (int32_t*)t;

    c->host_pack = (const char*)host_pack;
    c->slots_dev = (char*)device;
    for (int m = 0; m < 3; ++m) {
        c->slot0[m].seeds = (const uint16_t*)(c->slots_dev + off[3 * m]);
        c->slot0[m].coefs = (const uint16_t*)(c->slots_dev + off[3 * m + 1]);
        c->slot0[m].codes = (const uint8_t*)(c->slots_dev + off[3 * m + 2]);
        c->slot0[m].exp_bias = exp_bias + (int64_t)m * E;
    }
    c->slot_map_dev = (int32_t*)(c->slots_dev + up256(c->record * (size_t)S));
    clear_tables(c);
    c->magic = kMagic;
    return SEEDMM_OK;
}

int seedmm_cache_reset(seedmm_cache* c) {
    if (!valid(c)) return SEEDMM_EINVAL;
    clear_tables(c);
    memset(c->stats, 0, sizeof(c->stats));
    c->step = 0;
    return SEEDMM_OK;
}

int seedmm_cache_plan(seedmm_cache* c, const int32_t* ids, int T, int top_k, int32_t* loads,
                      int* n_loads) {
    if (!valid(c) || T < 0 || top_k < 1 || top_k > c->E) return SEEDMM_EINVAL;
    if (T > 0 && !ids) return SEEDMM_EINVAL;
    const int64_t pairs = (int64_t)T * top_k;
    for (int64_t i = 0; i < pairs; ++i)
        if (ids[i] < 0 || ids[i] >= c->E) return SEEDMM_EINVAL;
    memset(c->used, 0, (size_t)c->E);
    int distinct = 0;
    for (int64_t i = 0; i < pairs; ++i)
        if (!c->used[ids[i]]) {
            c->used[ids[i]] = 1;
            ++distinct;
        }
    if (distinct > c->S) return SEEDMM_ECAPACITY;

    const uint64_t now = ++c->step;
    int hits = 0, n = 0;
    for (int e = 0; e < c->E; ++e)
        if (c->used[e] && c->slot_of[e] >= 0) {
            c->last_use[c->slot_of[e]] = now;
            ++hits;
        }
    for (int e = 0; e < c->E; ++e) {
        if (!c->used[e] || c->slot_of[e] >= 0) continue;
        int v = -1;
        for (int s = 0; s < c->S && v < 0; ++s)
            if (c->expert_of[s] < 0) v = s;
        if (v < 0)
            for (int s = 0; s < c->S; ++s)
                if (c->last_use[s] < now && (v < 0 || c->last_use[s] < c->last_use[v])) v = s;
        // distinct <= S guarantees a slot that this call does not use
        if (c->expert_of[v] >= 0) c->slot_of[c->expert_of[v]] = -1;
        c->expert_of[v] = e;
        c->slot_of[e] = v;
        c->last_use[v] = now;
        if (loads) {
            loads[2 * n] = e;
            loads[2 * n + 1] = v;
        }
        ++n;
    }
    if (n_loads) *n_loads = n;
    c->stats[0] += 1;
    c->stats[1] += (uint64_t)distinct;
    c->stats[2] += (uint64_t)hits;
    c->stats[3] += (uint64_t)n;
    c->stats[4] += (uint64_t)n * c->record;
    return SEEDMM_OK;
}

int seedmm_cache_moe(seedmm_cache* c, const int32_t* ids_host, const int32_t* topk_ids,
                     const float* topk_w, int T, int top_k, const void* x, float* y,
                     void* workspace, size_t workspace_bytes, void* hip_stream) {
    // every argument is checked before the plan changes the state
    if (!valid(c) || T < 0 || top_k < 1 || top_k > c->E || top_k > 64) return SEEDMM_EINVAL;
    if (T > 0) {
        if (!ids_host || !topk_ids || !topk_w || !x || !y) return SEEDMM_EINVAL;
        if (((uintptr_t)x & 15) != 0 || ((uintptr_t)y & 15) != 0) return SEEDMM_EALIGN;
        const size_t need = seedmm_moe_workspace_bytes(T, top_k, c->E, c->H, c->I);
        if (!workspace || need == 0 || workspace_bytes < need) return SEEDMM_EWORKSPACE;
        if (((uintptr_t)workspace & 15) != 0) return SEEDMM_EALIGN;
    }
    int n = 0;
    int st = seedmm_cache_plan(c, ids_host, T, top_k, c->loads, &n);
    if (st != SEEDMM_OK) return st;
    if (T == 0) return SEEDMM_OK;
    hipStream_t s = (hipStream_t)hip_stream;

    auto fail = [&]() {
        clear_tables(c);
        return SEEDMM_EHIP;
    };
    // one host-to-device copy per loaded expert: its whole record into its slot
    for (int i = 0; i < n; ++i) {
        const int e = c->loads[2 * i], v = c->loads[2 * i + 1];
        if (hipMemcpyAsync(c->slots_dev + c->record * (size_t)v, c->host_pack + c->record * (size_t)e,
                           c->record, hipMemcpyHostToDevice, s) != hipSuccess)
            return fail();
    }
    // the device map: every entry slot 0 once, then each loaded expert's slot.  Entries
    // of experts that are not resident are never read (the kernels look up only this
    // call's experts); they always hold some slot in [0, S), so even a device id that
    // disagreed with the host's would read inside the slots.
    if (!c->device_map_valid) {
        hipLaunchKernelGGL(k_map_fill, dim3((c->E + 255) / 256), dim3(256), 0, s, c->slot_map_dev,
                           c->E, 0);
        if (hipGetLastError() != hipSuccess) return fail();
        // after a fill every resident expert is written again
        n = 0;
        for (int e = 0; e < c->E; ++e)
            if (c->slot_of[e] >= 0) {
                c->loads[2 * n] = e;
                c->loads[2 * n + 1] = c->slot_of[e];
                ++n;
            }
        c->device_map_valid = true;
    }
    MapUpdate u;
    u.n = 0;
    auto flush = [&]() {
        if (u.n == 0) return true;
        hipLaunchKernelGGL(k_map_update, dim3(1), dim3(256), 0, s, c->slot_map_dev, u);
        u.n = 0;
        return hipGetLastError() == hipSuccess;
    };
    for (int i = 0; i < n; ++i) {
        if (u.n == kUpd && !flush()) return fail();
        u.idx[u.n] = c->loads[2 * i];
        u.val[u.n] = c->loads[2 * i + 1];
        ++u.n;
    }
    if (!flush()) return fail();

    st = seedmm_layer::moe_run(topk_ids, topk_w, T, top_k, x, y, c->E, c->H, c->I, c->P,
                               nullptr, c->slot0[0], c->slot0[1], c->slot0[2], workspace,
                               workspace_bytes, hip_stream, nullptr, c->slot_map_dev,
                               (int64_t)c->record, nullptr);
    if (st == SEEDMM_EHIP) return fail();
    return st;
}

int seedmm_cache_stats(const seedmm_cache* c, uint64_t out[5]) {
    if (!valid(c) || !out) return SEEDMM_EINVAL;
    for (int i = 0; i < 5; ++i) out[i] = c->stats[i];
    return SEEDMM_OK;
}

}  // extern "C"
