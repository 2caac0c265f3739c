// Host side of regen_attn: argument checking, rotary tables, workspace,
// launches. The C ABI is declared (with its contract) in include/regen_attn.h.
#include "regen_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "attention.hpp"
#include "cross.hpp"
#include "gemm.hpp"
#include "layout.hpp"
#include "probe.hpp"

namespace {

constexpr uint32_t kKnownFlags = REGEN_ATTN_NO_ROPE | REGEN_ATTN_PROFILE | REGEN_ATTN_TOKEN_MAJOR;
// Attention kernel shape: NW waves of 32 query rows, BN-key blocks.
constexpr int kNW = 8, kBM = kNW * 32, kBN = 64;
constexpr int64_t kMaxTokens = int64_t(1) << 30;

thread_local std::string g_last_error;

// Live handles. A handle is looked up here before it is dereferenced, so a
// destroyed or foreign pointer is rejected instead of being read.
std::mutex g_live_mu;
std::unordered_set<const void*> g_live;

bool is_live(const void* h) {
    std::lock_guard<std::mutex> lk(g_live_mu);
    return g_live.count(h) != 0;
}

regen_status fail(regen_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

regen_status fail_hip(hipError_t e, const char* what) {
    std::string m = what;
    m += ": ";
    m += hipGetErrorString(e);
    return fail(REGEN_ERR_HIP, m);
}

// Fully resolved problem: defaults applied, all fields checked.
struct Problem {
    int heads, head_dim, T, H, W;
    int pairs[3];
    double base;
    float scale;
    uint32_t flags;
    int64_t tokens, tokens_pad;
    int n_qtiles, nkv;
    int64_t units;  // heads * n_qtiles * nkv
};

regen_status resolve(const regen_attn_desc* d, Problem* p) {
    if (!d) return fail(REGEN_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (d->struct_size != sizeof(regen_attn_desc))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "desc->struct_size does not match this library");
    if (d->heads < 1) return fail(REGEN_ERR_INVALID_ARGUMENT, "heads must be >= 1");
    if (d->grid_t < 1 || d->grid_h < 1 || d->grid_w < 1)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "grid_t, grid_h, grid_w must be >= 1");
    if (d->flags & ~kKnownFlags) return fail(REGEN_ERR_INVALID_ARGUMENT, "unknown flag bits");
    if (!(d->rope_base >= 0.0f) || !std::isfinite(d->rope_base))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "rope_base must be > 0 (or 0 for the default)");
    if (!(d->sm_scale >= 0.0f) || !std::isfinite(d->sm_scale))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "sm_scale must be > 0 (or 0 for the default)");
    if (d->head_dim <= 0 || d->head_dim % 2 != 0)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "head_dim must be a positive even number");
    const int half = d->head_dim / 2;
    int pt = d->pairs_t, ph = d->pairs_h, pw = d->pairs_w;
    if (pt == 0 && ph == 0 && pw == 0) {
        ph = pw = half / 3;
        pt = half - 2 * ph;
    } else if (pt < 1 || ph < 1 || pw < 1 || pt + ph + pw != half) {
        return fail(REGEN_ERR_INVALID_ARGUMENT,
                    "pairs_t/h/w must each be >= 1 and sum to head_dim/2 (or all be 0)");
    }
    const int64_t tokens = int64_t(d->grid_t) * d->grid_h * d->grid_w;
    if (tokens > kMaxTokens) return fail(REGEN_ERR_INVALID_ARGUMENT, "too many tokens (> 2^30)");
    if (int64_t(d->heads) * tokens * d->head_dim > (int64_t(1) << 40))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "tensor too large");
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(REGEN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    // One head's rotated K (and transposed V) is addressed through a buffer
    // resource with 32-bit offsets.
    if ((tokens + regen::kPrepKeys - 1) / regen::kPrepKeys * regen::kPrepKeys * d->head_dim * 2 >=
        (int64_t(1) << 31))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "too many tokens for one head (K workspace >= 2^31 bytes)");
    p->heads = d->heads;
    p->head_dim = d->head_dim;
    p->T = d->grid_t;
    p->H = d->grid_h;
    p->W = d->grid_w;
    p->pairs[0] = pt;
    p->pairs[1] = ph;
    p->pairs[2] = pw;
    p->base = d->rope_base > 0.0f ? double(d->rope_base) : 10000.0;
    p->scale = d->sm_scale > 0.0f ? d->sm_scale : float(1.0 / std::sqrt(double(d->head_dim)));
    p->flags = d->flags;
    p->tokens = tokens;
    p->tokens_pad = (tokens + regen::kPrepKeys - 1) / regen::kPrepKeys * regen::kPrepKeys;
    p->n_qtiles = int((tokens + kBM - 1) / kBM);
    p->nkv = int((tokens + kBN - 1) / kBN);
    p->units = int64_t(p->heads) * p->n_qtiles * p->nkv;
    // The attention schedule numbers (query tile, key block) pairs in 31 bits.
    if (p->units >= (int64_t(1) << 31))
        return fail(REGEN_ERR_INVALID_ARGUMENT,
                    "too many (query tile, key block) pairs: heads * ceil(tokens/256) * "
                    "ceil(tokens/64) must stay below 2^31");
    return REGEN_OK;
}

// Rotary geometry of p (axis extents, pairs, table offsets); returns the
// number of table entries, T P_t + H P_h + W P_w.
int64_t rope_geometry(const Problem& p, regen::RopeGeom* geo) {
    geo->T = p.T;
    geo->H = p.H;
    geo->W = p.W;
    const int extent[3] = {p.T, p.H, p.W};
    int64_t off = 0;
    for (int a = 0; a < 3; ++a) {
        geo->pairs[a] = p.pairs[a];
        geo->off[a] = int(std::min<int64_t>(off, INT32_MAX));
        off += int64_t(extent[a]) * p.pairs[a];
    }
    return off;
}

size_t workspace_bytes(const Problem& p) {
    // Kr and Vt, bf16 each.
    return size_t(2) * size_t(p.heads) * size_t(p.tokens_pad) * size_t(p.head_dim) * 2;
}

}  // namespace

// Events of one profiled forward: before the first kernel, between
// consecutive kernels, after the last.
struct ProfRecord {
    hipEvent_t ev[4];
};

// One set of the device buffers a call writes besides its output. A handle
// holds kSlots of them, so that calls issued on different streams can run at
// the same time; acquire_slot() picks one per call and fences it with its
// event, which makes a handle read-only from the caller's point of view.
struct Slot {
    uint16_t* kr;        // rotated K, [heads][Npad/64] fragment-ordered tiles
    uint16_t* vt;        // transposed V, same layout
    uint16_t* part_o;    // split-tile O / l, bf16 [2P][BM][D]
    float* part_ml;      // split-tile (m, l)      [2P][BM][2]
    int* cnt;            // leftover piece counter (zeroed by the K pass)
    uint16_t* qkv;       // attention blocks only: projection output [N][3 hidden]
    uint16_t* attn_out;  // attention blocks only: attention output  [N][hidden]
    hipEvent_t done;     // recorded after the last kernel of every call using the slot
    hipStream_t last;    // the stream of that call
    bool used;
    uint64_t stamp;      // order of last use
};
constexpr int kSlots = 2;
constexpr int kPieceBlocks = 6;  // key blocks per claimed leftover piece (at least)

struct regen_attn {
    int device;
    std::mutex mu;  // guards the slots and the profiling lists
    std::vector<ProfRecord> prof_pending;  // recorded, not yet read
    std::vector<ProfRecord> prof_free;     // created, reusable
    Problem p;
    regen::RopeGeom geo;
    float2* d_tab;     // rotary (cos, sin) per axis
    float2* d_tab_id;  // the same table with every angle 0 (unrotated calls)
    int P;             // persistent attention workgroups
    int Pc;            // cross_attn_kernel workgroups (one round of resident slots)
    Slot slot[kSlots];
    uint64_t stamp;
};

namespace {

template <int D>
regen_status occupancy(int* blocks_per_cu, int* cross_blocks_per_cu) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, regen::attn_fwd_kernel<D, kBN, kNW>, kNW * 64, 0);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            cross_blocks_per_cu, regen::cross_attn_kernel<D, kNW, true>, kNW * 64, 0);
    if (e != hipSuccess) return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    if (*blocks_per_cu < 1) *blocks_per_cu = 1;
    if (*cross_blocks_per_cu < 1) *cross_blocks_per_cu = 1;
    return REGEN_OK;
}

// Release a handle's device memory and events (each pointer may be NULL) and
// the handle. Waits first for the last call on each slot.
void free_handle(regen_attn* h) {
    int cur = 0;
    const bool switched = hipGetDevice(&cur) == hipSuccess && cur != h->device &&
                          hipSetDevice(h->device) == hipSuccess;
    for (Slot& sl : h->slot)
        if (sl.done && sl.used) (void)hipEventSynchronize(sl.done);
    if (h->d_tab) (void)hipFree(h->d_tab);
    for (Slot& sl : h->slot) {
        for (void* ptr : {(void*)sl.kr, (void*)sl.vt, (void*)sl.part_o, (void*)sl.part_ml, (void*)sl.cnt,
                          (void*)sl.qkv, (void*)sl.attn_out})
            if (ptr) (void)hipFree(ptr);
        if (sl.done) (void)hipEventDestroy(sl.done);
    }
    for (auto* list : {&h->prof_pending, &h->prof_free})
        for (ProfRecord& r : *list)
            for (hipEvent_t ev : r.ev) (void)hipEventDestroy(ev);
    if (switched) (void)hipSetDevice(cur);
    delete h;
}

// The slot for a call on stream st (h->mu held): the one this stream used
// last (stream order already puts the new call after that one), else one
// never used, else the least recently used one, after making st wait for
// the last call that used it.
regen_status acquire_slot(regen_attn* h, hipStream_t st, Slot** out) {
    Slot* pick = nullptr;
    for (Slot& sl : h->slot)
        if (sl.used && sl.last == st) {
            pick = &sl;
            break;
        }
    if (!pick)
        for (Slot& sl : h->slot)
            if (!sl.used) {
                pick = &sl;
                break;
            }
    if (!pick) {
        pick = &h->slot[0];
        for (Slot& sl : h->slot)
            if (sl.stamp < pick->stamp) pick = &sl;
        const hipError_t e = hipStreamWaitEvent(st, pick->done, 0);
        if (e != hipSuccess) return fail_hip(e, "hipStreamWaitEvent");
    }
    *out = pick;
    return REGEN_OK;
}

// After a call's kernels are enqueued on st (h->mu held).
regen_status release_slot(regen_attn* h, Slot* sl, hipStream_t st) {
    const hipError_t e = hipEventRecord(sl->done, st);
    if (e != hipSuccess) return fail_hip(e, "hipEventRecord");
    sl->last = st;
    sl->used = true;
    sl->stamp = ++h->stamp;
    return REGEN_OK;
}

}  // namespace

extern "C" {

const char* regen_attn_status_string(regen_status s) {
    switch (s) {
        case REGEN_OK: return "REGEN_OK";
        case REGEN_ERR_INVALID_ARGUMENT: return "REGEN_ERR_INVALID_ARGUMENT";
        case REGEN_ERR_UNSUPPORTED: return "REGEN_ERR_UNSUPPORTED";
        case REGEN_ERR_NO_DEVICE: return "REGEN_ERR_NO_DEVICE";
        case REGEN_ERR_OUT_OF_MEMORY: return "REGEN_ERR_OUT_OF_MEMORY";
        case REGEN_ERR_HIP: return "REGEN_ERR_HIP";
    }
    return "REGEN_ERR_UNKNOWN";
}

const char* regen_attn_last_error(void) { return g_last_error.c_str(); }

size_t regen_attn_workspace_size(const regen_attn_desc* desc) {
    Problem p;
    std::string saved = g_last_error;
    regen_status s = resolve(desc, &p);
    g_last_error = saved;
    return s == REGEN_OK ? workspace_bytes(p) : 0;
}

regen_status regen_attn_create(const regen_attn_desc* desc, regen_attn_t* out) {
    g_last_error.clear();
    if (!out) return fail(REGEN_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    Problem p;
    regen_status s = resolve(desc, &p);
    if (s != REGEN_OK) return s;

    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return fail(REGEN_ERR_NO_DEVICE, "no HIP device is available");
    }
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return fail_hip(e, "hipGetDevice");
    hipDeviceProp_t prop;
    if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess)
        return fail_hip(e, "hipGetDeviceProperties");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(REGEN_ERR_UNSUPPORTED,
                    std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950");

    // Rotary tables in fp64, stored as fp32 (cos, sin).
    regen::RopeGeom geo;
    const int64_t entries = rope_geometry(p, &geo);
    if (entries >= (int64_t(1) << 31))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "rotary table too large (grid extent x pairs >= 2^31)");
    const int extent[3] = {p.T, p.H, p.W};
    std::vector<float2> tab(entries);
    const bool rope = !(p.flags & REGEN_ATTN_NO_ROPE);
    for (int a = 0; a < 3; ++a)
        for (int pos = 0; pos < extent[a]; ++pos)
            for (int j = 0; j < p.pairs[a]; ++j) {
                const double theta = std::pow(p.base, -double(j) / double(p.pairs[a]));
                const double phi = double(pos) * theta;
                float2 cs;
                cs.x = rope ? float(std::cos(phi)) : 1.0f;
                cs.y = rope ? float(std::sin(phi)) : 0.0f;
                tab[geo.off[a] + pos * p.pairs[a] + j] = cs;
            }

    regen_attn* h = new (std::nothrow) regen_attn();
    if (!h) return fail(REGEN_ERR_OUT_OF_MEMORY, "host allocation of the handle failed");
    h->device = dev;
    h->p = p;
    h->geo = geo;
    h->d_tab = h->d_tab_id = nullptr;
    h->stamp = 0;
    for (Slot& sl : h->slot) sl = Slot{};
    int per_cu = 1, cross_per_cu = 1;
    s = p.head_dim == 128 ? occupancy<128>(&per_cu, &cross_per_cu) : occupancy<64>(&per_cu, &cross_per_cu);
    if (s != REGEN_OK) {
        delete h;
        return s;
    }
    const int64_t slots = int64_t(per_cu) * prop.multiProcessorCount;
    h->P = int(slots < p.units ? slots : p.units);
    h->Pc = cross_per_cu * prop.multiProcessorCount;

    const size_t tab_bytes = tab.size() * sizeof(float2);
    const size_t half_ws = workspace_bytes(p) / 2;
    const size_t part_o_bytes = size_t(2) * h->P * kBM * p.head_dim * sizeof(uint16_t);
    const size_t part_ml_bytes = size_t(2) * h->P * kBM * 2 * sizeof(float);
    e = hipMalloc(&h->d_tab, 2 * tab_bytes);
    for (Slot& sl : h->slot) {
        if (e == hipSuccess) e = hipMalloc(&sl.kr, half_ws);
        if (e == hipSuccess) e = hipMalloc(&sl.vt, half_ws);
        if (e == hipSuccess) e = hipMalloc(&sl.part_o, part_o_bytes);
        if (e == hipSuccess) e = hipMalloc(&sl.part_ml, part_ml_bytes);
        if (e == hipSuccess) e = hipMalloc(&sl.cnt, sizeof(int));
        if (e == hipSuccess) e = hipEventCreateWithFlags(&sl.done, hipEventDisableTiming);
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        free_handle(h);
        return fail(e == hipErrorOutOfMemory ? REGEN_ERR_OUT_OF_MEMORY : REGEN_ERR_HIP,
                    std::string("device allocation failed: ") + hipGetErrorString(e));
    }
    h->d_tab_id = h->d_tab + tab.size();
    tab.resize(2 * tab.size(), float2{1.0f, 0.0f});
    if ((e = hipMemcpy(h->d_tab, tab.data(), 2 * tab_bytes, hipMemcpyHostToDevice)) != hipSuccess) {
        free_handle(h);
        return fail_hip(e, "hipMemcpy of the rotary table");
    }
    {
        std::lock_guard<std::mutex> lk(g_live_mu);
        g_live.insert(h);
    }
    *out = h;
    return REGEN_OK;
}

}  // extern "C"

namespace {

// Overlap test of two byte ranges [a, a + na) and [b, b + nb).
bool overlaps(uintptr_t a, uintptr_t na, uintptr_t b, uintptr_t nb) {
    return a < b + nb && b < a + na;
}

// Element strides of (head, token) in q, k/v and o.
struct Strides {
    long long qh, qn, kh, kn, oh, on;
};

// What one call's kernels need besides its arguments: the problem, the
// rotary tables, the workgroup counts and the buffers of one slot.
struct Ctx {
    const Problem* p;
    const regen::RopeGeom* geo;
    const float2* tab;
    const float2* tab_id;
    int P, Pc;
    uint16_t* kr;
    uint16_t* vt;
    uint16_t* part_o;
    float* part_ml;
    int* cnt;
};

regen_status enqueue(const Ctx& c, const void* q, int64_t q_begin, int64_t nq, const void* k,
                     const void* v, int64_t kv_begin, int64_t nk, void* o, float* lse, void* stream,
                     bool cross, const Strides& sd, ProfRecord* rec);

// Checks of one call's ranges and pointers against problem p.
regen_status check_call(const Problem& p, const void* q, int64_t q_begin, int64_t nq, const void* k,
                        const void* v, int64_t kv_begin, int64_t nk, const void* o, const float* lse,
                        bool cross) {
    if (!q || !k || !v || !o) return fail(REGEN_ERR_INVALID_ARGUMENT, "q, k, v, o must be non-NULL");
    if (q_begin < 0 || nq < 1 || q_begin + nq > p.tokens)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "query range outside [0, grid_t*grid_h*grid_w)");
    if (cross) {
        if (nk < 1 || nk > p.tokens)
            return fail(REGEN_ERR_INVALID_ARGUMENT, "ctx_len must be in [1, grid_t*grid_h*grid_w]");
    } else if (kv_begin < 0 || nk < 1 || kv_begin + nk > p.tokens) {
        return fail(REGEN_ERR_INVALID_ARGUMENT, "key range outside [0, grid_t*grid_h*grid_w)");
    }
    const uintptr_t ptrs[4] = {uintptr_t(q), uintptr_t(k), uintptr_t(v), uintptr_t(o)};
    for (uintptr_t a : ptrs)
        if (a % 16 != 0) return fail(REGEN_ERR_INVALID_ARGUMENT, "q, k, v, o must be 16-byte aligned");
    if (lse && uintptr_t(lse) % 4 != 0)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    const uintptr_t row = uintptr_t(p.heads) * uintptr_t(p.head_dim) * 2;
    const uintptr_t qbytes = row * uintptr_t(nq), kbytes = row * uintptr_t(nk);
    const uintptr_t lbytes = uintptr_t(p.heads) * uintptr_t(nq) * 4;
    if (overlaps(ptrs[3], qbytes, ptrs[0], qbytes) || overlaps(ptrs[3], qbytes, ptrs[1], kbytes) ||
        overlaps(ptrs[3], qbytes, ptrs[2], kbytes))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "o overlaps q, k or v");
    if (lse && (overlaps(uintptr_t(lse), lbytes, ptrs[0], qbytes) ||
                overlaps(uintptr_t(lse), lbytes, ptrs[1], kbytes) ||
                overlaps(uintptr_t(lse), lbytes, ptrs[2], kbytes) ||
                overlaps(uintptr_t(lse), lbytes, ptrs[3], qbytes)))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "lse overlaps q, k, v or o");
    return REGEN_OK;
}

// Strides of the caller's q, k, v, o under the problem's layout flag.
Strides caller_strides(const Problem& p, int64_t nq, int64_t nk) {
    const bool tm = (p.flags & REGEN_ATTN_TOKEN_MAJOR) != 0;
    const long long D = p.head_dim;
    Strides sd;
    sd.qh = sd.oh = tm ? D : nq * D;
    sd.qn = sd.on = tm ? p.heads * D : D;
    sd.kh = tm ? D : nk * D;
    sd.kn = tm ? p.heads * D : D;
    return sd;
}

Ctx handle_ctx(const regen_attn* h, const Slot* sl) {
    return Ctx{&h->p, &h->geo, h->d_tab, h->d_tab_id, h->P, h->Pc, sl->kr, sl->vt, sl->part_o,
               sl->part_ml, sl->cnt};
}

// One profiling record of handle h (h->mu held), or NULL for an unprofiled handle.
regen_status prof_record(regen_attn* h, ProfRecord** out) {
    *out = nullptr;
    if (!(h->p.flags & REGEN_ATTN_PROFILE)) return REGEN_OK;
    ProfRecord rec{};
    if (!h->prof_free.empty()) {
        rec = h->prof_free.back();
        h->prof_free.pop_back();
    } else {
        for (int i = 0; i < 4; ++i) {
            const hipError_t e = hipEventCreate(&rec.ev[i]);
            if (e != hipSuccess) {
                for (int j = 0; j < i; ++j) (void)hipEventDestroy(rec.ev[j]);
                return fail_hip(e, "hipEventCreate");
            }
        }
    }
    h->prof_pending.push_back(rec);
    *out = &h->prof_pending.back();
    return REGEN_OK;
}

// Enqueue `body(ctx, rec)` on stream st with one of handle h's slots.
template <typename F>
regen_status with_slot(regen_attn* h, void* stream, F body) {
    int cur = -1;
    const hipError_t ge = hipGetDevice(&cur);
    if (ge != hipSuccess) return fail_hip(ge, "hipGetDevice");
    if (cur != h->device)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "the current HIP device is not the handle's device");
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lk(h->mu);
    Slot* sl = nullptr;
    regen_status s = acquire_slot(h, st, &sl);
    if (s != REGEN_OK) return s;
    ProfRecord* rec = nullptr;
    s = prof_record(h, &rec);
    if (s != REGEN_OK) return s;
    s = body(sl, rec);
    const regen_status r = release_slot(h, sl, st);
    return s != REGEN_OK ? s : r;
}

// One attention call: query tokens [q_begin, q_begin + nq) against key
// tokens [kv_begin, kv_begin + nk) of the handle's window.
regen_status launch(regen_attn_t h, const void* q, int64_t q_begin, int64_t nq, const void* k,
                    const void* v, int64_t kv_begin, int64_t nk, void* o, float* lse,
                    void* stream, bool cross = false) {
    if (!h || !is_live(h)) return fail(REGEN_ERR_INVALID_ARGUMENT, "handle is NULL or not live");
    const Problem& p = h->p;
    regen_status s = check_call(p, q, q_begin, nq, k, v, kv_begin, nk, o, lse, cross);
    if (s != REGEN_OK) return s;
    const Strides sd = caller_strides(p, nq, nk);
    return with_slot(h, stream, [&](Slot* sl, ProfRecord* rec) {
        return enqueue(handle_ctx(h, sl), q, q_begin, nq, k, v, kv_begin, nk, o, lse, stream, cross, sd,
                       rec);
    });
}

// Schedule of the persistent attention kernel over P workgroups for one
// call (see regen::Sched). False if the call's unit count needs more than
// 31 bits.
bool make_sched(int heads, int64_t nq, int64_t nk, int P, regen::Sched* sc, int64_t* rem_tiles) {
    const int64_t n_qtiles = (nq + kBM - 1) / kBM, nkv = (nk + kBN - 1) / kBN;
    const int64_t tiles = int64_t(heads) * n_qtiles;
    if (tiles * nkv >= (int64_t(1) << 31)) return false;
    sc->n_qtiles = int(n_qtiles);
    sc->nkv = int(nkv);
    sc->P = P;
    sc->full = int(tiles / P);
    *rem_tiles = tiles - int64_t(sc->full) * P;
    sc->rem_units = int(*rem_tiles * nkv);
    sc->Prem = sc->rem_units < P ? (sc->rem_units > 0 ? sc->rem_units : 1) : P;
    sc->rem_q = sc->rem_units / sc->Prem;
    sc->rem_r = sc->rem_units % sc->Prem;
    // A small leftover after whole-tile passes (at most 8 key blocks per
    // workgroup) is cut into pieces of at least kPieceBlocks key blocks that
    // workgroups claim as they finish, at most 2P of them (one partial slot
    // each). Pieces of 3 / 6 / 12 blocks measured 618.8 / 616.3 / 615.5 us
    // per 12 x 10920 call against 628.0 for the static split; larger pieces
    // cost more where the XCDs' clocks happen to agree. Only for long key
    // runs (at least 16 pieces' worth per tile): with short ones a workgroup's
    // whole share is a few blocks, the clocks' spread is a fraction of a
    // block, and a claimed piece costs more than the static split (512 keys:
    // 51 -> 59 us).
    sc->dyn = 0;
    sc->ppt = 1;
    sc->npieces = 0;
    if (sc->full >= 1 && *rem_tiles > 0 && sc->rem_units <= int64_t(8) * P && nkv >= 16 * kPieceBlocks) {
        const int64_t ppt =
            std::min<int64_t>(std::max<int64_t>(nkv / kPieceBlocks, 1), 2 * int64_t(P) / *rem_tiles);
        sc->dyn = 1;
        sc->ppt = int(ppt);
        sc->npieces = int(*rem_tiles * ppt);
    }
    return true;
}

// Enqueue the kernels of one call whose arguments have been checked; with
// rec, record its events around them.
regen_status enqueue(const Ctx& c, const void* q, int64_t q_begin, int64_t nq, const void* k,
                     const void* v, int64_t kv_begin, int64_t nk, void* o, float* lse, void* stream,
                     bool cross, const Strides& sd, ProfRecord* rec) {
    const Problem& p = *c.p;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int Nq = int(nq), Nk = int(nk);
    const int Npad = int((nk + regen::kPrepKeys - 1) / regen::kPrepKeys * regen::kPrepKeys);
    const float c2 = p.scale * 1.4426950408889634f;

    dim3 pgrid(unsigned(Npad / regen::kPrepBlock), unsigned(p.heads), unsigned(p.head_dim / regen::kPrepDims));
    // A K pass of fewer than 8 blocks per CU stores nontemporally.
    const bool kp_nt = int64_t(pgrid.x) * pgrid.y * pgrid.z < int64_t(8) * c.P;
    regen::Sched sc;
    int64_t rem_tiles = 0;
    if (!make_sched(p.heads, nq, nk, c.P, &sc, &rem_tiles))
        return fail(REGEN_ERR_INVALID_ARGUMENT,
                    "too many (query tile, key block) pairs for one call (heads * ceil(q/256) * "
                    "ceil(k/64) must stay below 2^31)");
    // Tiles split many ways merge with 4 waves per row, others with one.
    const bool mw4 = sc.dyn ? sc.ppt >= 8 : sc.Prem >= 8 * rem_tiles;
    const dim3 mgrid{unsigned(rem_tiles), unsigned(mw4 ? kBM : kBM / 16), 1u};
    const uint16_t* q16 = static_cast<const uint16_t*>(q);
    const uint16_t* k16 = static_cast<const uint16_t*>(k);
    const uint16_t* v16 = static_cast<const uint16_t*>(v);
    uint16_t* o16 = static_cast<uint16_t*>(o);
    const int q_off = int(q_begin), k_off = int(kv_begin);
    // Cross-attention rotates nothing: the identity table.
    const float2* tab = cross ? c.tab_id : c.tab;
    const regen::RopeGeom& geo = *c.geo;
    const long long qh = sd.qh, qn = sd.qn, kh = sd.kh, kn = sd.kn, oh = sd.oh, on = sd.on;

    const bool prof = rec != nullptr;
    if (prof) (void)hipEventRecord(rec->ev[0], st);
    auto mark = [&](int i) {
        if (prof) (void)hipEventRecord(rec->ev[i], st);
    };

    // A short context stays in LDS: one kernel, one pass over the queries.
    // Its buffer resources take byte offsets below 2^31 into one head of q,
    // o, lse and the context (2^31 marks an access to drop).
    const int64_t span_q = ((nq - 1) * std::max(qn, on) + p.head_dim) * 2;
    const bool short_ctx = cross && nk <= regen::kCrossMaxKeys && nk * kn * 2 < (int64_t(1) << 31) &&
                           span_q < (int64_t(1) << 31) && nq * 4 < (int64_t(1) << 31);
    const int64_t cross_units = int64_t(p.heads) * ((nq + 31) / 32);
    const dim3 cgrid{unsigned(std::min<int64_t>(c.Pc, cross_units)), 1u, 1u};
    if (short_ctx) {
        mark(1);
        if (p.head_dim == 128) {
            if (lse)
                hipLaunchKernelGGL((regen::cross_attn_kernel<128, kNW, true>), cgrid, dim3(kNW * 64), 0, st,
                                   q16, k16, v16, o16, lse, Nq, Nk, qh, qn, kh, kn, oh, on, p.heads, c2);
            else
                hipLaunchKernelGGL((regen::cross_attn_kernel<128, kNW, false>), cgrid, dim3(kNW * 64), 0, st,
                                   q16, k16, v16, o16, lse, Nq, Nk, qh, qn, kh, kn, oh, on, p.heads, c2);
        } else {
            if (lse)
                hipLaunchKernelGGL((regen::cross_attn_kernel<64, kNW, true>), cgrid, dim3(kNW * 64), 0, st,
                                   q16, k16, v16, o16, lse, Nq, Nk, qh, qn, kh, kn, oh, on, p.heads, c2);
            else
                hipLaunchKernelGGL((regen::cross_attn_kernel<64, kNW, false>), cgrid, dim3(kNW * 64), 0, st,
                                   q16, k16, v16, o16, lse, Nq, Nk, qh, qn, kh, kn, oh, on, p.heads, c2);
        }
        mark(2);
    } else if (p.head_dim == 128) {
        if (kp_nt)
            hipLaunchKernelGGL((regen::rope_k_vt_kernel<128, true>), pgrid, dim3(256), 0, st, k16, v16, c.kr,
                               c.vt, tab, geo, Nk, Npad, k_off, kh, kn, sc.dyn ? c.cnt : nullptr);
        else
            hipLaunchKernelGGL((regen::rope_k_vt_kernel<128, false>), pgrid, dim3(256), 0, st, k16, v16, c.kr,
                               c.vt, tab, geo, Nk, Npad, k_off, kh, kn, sc.dyn ? c.cnt : nullptr);
        mark(1);
        hipLaunchKernelGGL((regen::attn_fwd_kernel<128, kBN, kNW>), dim3(c.P), dim3(kNW * 64), 0,
                           st, q16, c.kr, c.vt, o16, lse, tab, geo, Nq, Nk, Npad,
                           q_off, qh, qn, oh, on, sc, c2, int(!cross), c.part_o, c.part_ml, c.cnt);
        mark(2);
        if (rem_tiles > 0) {
            if (mw4)
                hipLaunchKernelGGL((regen::merge_kernel<128, kNW, 4>), mgrid, dim3(256), 0, st, o16,
                                   lse, c.part_o, c.part_ml, Nq, sc, oh, on);
            else
                hipLaunchKernelGGL((regen::merge_kernel<128, kNW, 1>), mgrid, dim3(256), 0, st, o16,
                                   lse, c.part_o, c.part_ml, Nq, sc, oh, on);
        }
    } else {
        hipLaunchKernelGGL((regen::rope_k_vt_kernel<64, false>), pgrid, dim3(256), 0, st, k16, v16, c.kr,
                           c.vt, tab, geo, Nk, Npad, k_off, kh, kn, sc.dyn ? c.cnt : nullptr);
        mark(1);
        hipLaunchKernelGGL((regen::attn_fwd_kernel<64, kBN, kNW>), dim3(c.P), dim3(kNW * 64), 0,
                           st, q16, c.kr, c.vt, o16, lse, tab, geo, Nq, Nk, Npad,
                           q_off, qh, qn, oh, on, sc, c2, int(!cross), c.part_o, c.part_ml, c.cnt);
        mark(2);
        if (rem_tiles > 0) {
            if (mw4)
                hipLaunchKernelGGL((regen::merge_kernel<64, kNW, 4>), mgrid, dim3(256), 0, st, o16,
                                   lse, c.part_o, c.part_ml, Nq, sc, oh, on);
            else
                hipLaunchKernelGGL((regen::merge_kernel<64, kNW, 1>), mgrid, dim3(256), 0, st, o16,
                                   lse, c.part_o, c.part_ml, Nq, sc, oh, on);
        }
    }
    hipError_t e = hipGetLastError();
    if (prof) (void)hipEventRecord(rec->ev[3], st);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    return REGEN_OK;
}

}  // namespace

extern "C" {

regen_status regen_attn_forward(regen_attn_t h, const void* q, const void* k, const void* v,
                                void* o, void* stream) {
    g_last_error.clear();
    if (!h || !is_live(h)) return fail(REGEN_ERR_INVALID_ARGUMENT, "handle is NULL or not live");
    return launch(h, q, 0, h->p.tokens, k, v, 0, h->p.tokens, o, nullptr, stream);
}

regen_status regen_attn_forward_range(regen_attn_t h, const void* q, int64_t q_begin,
                                      int64_t q_count, const void* k, const void* v,
                                      int64_t kv_begin, int64_t kv_count, void* o, float* lse,
                                      void* stream) {
    g_last_error.clear();
    return launch(h, q, q_begin, q_count, k, v, kv_begin, kv_count, o, lse, stream);
}

regen_status regen_attn_forward_cross(regen_attn_t h, const void* q, const void* k_ctx,
                                      const void* v_ctx, int64_t ctx_len, void* o, float* lse,
                                      void* stream) {
    g_last_error.clear();
    if (!h || !is_live(h)) return fail(REGEN_ERR_INVALID_ARGUMENT, "handle is NULL or not live");
    return launch(h, q, 0, h->p.tokens, k_ctx, v_ctx, 0, ctx_len, o, lse, stream, true);
}

regen_status regen_attn_merge(const void* const* o_parts, const float* const* lse_parts,
                              int nparts, int heads, int64_t rows, int head_dim, void* o,
                              float* lse, void* stream) {
    g_last_error.clear();
    if (!o_parts || !lse_parts || !o)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "o_parts, lse_parts and o must be non-NULL");
    if (nparts < 1 || nparts > regen::kMaxMergeParts)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "nparts must be in [1, 8]");
    if (heads < 1 || rows < 1) return fail(REGEN_ERR_INVALID_ARGUMENT, "heads and rows must be >= 1");
    if (head_dim != 64 && head_dim != 128)
        return fail(REGEN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    const int64_t total = int64_t(heads) * rows;
    if (total > (int64_t(1) << 40) / head_dim)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "tensor too large");
    const uintptr_t obytes = uintptr_t(total) * uintptr_t(head_dim) * 2;
    const uintptr_t lbytes = uintptr_t(total) * 4;
    if (uintptr_t(o) % 16 != 0 || (lse && uintptr_t(lse) % 4 != 0))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "o must be 16-byte and lse 4-byte aligned");
    regen::MergeParts mp{};
    for (int i = 0; i < nparts; ++i) {
        if (!o_parts[i] || !lse_parts[i])
            return fail(REGEN_ERR_INVALID_ARGUMENT, "a part pointer is NULL");
        if (uintptr_t(o_parts[i]) % 16 != 0 || uintptr_t(lse_parts[i]) % 4 != 0)
            return fail(REGEN_ERR_INVALID_ARGUMENT, "o parts must be 16-byte and lse parts 4-byte aligned");
        if (overlaps(uintptr_t(o), obytes, uintptr_t(o_parts[i]), obytes) ||
            overlaps(uintptr_t(o), obytes, uintptr_t(lse_parts[i]), lbytes) ||
            (lse && (overlaps(uintptr_t(lse), lbytes, uintptr_t(o_parts[i]), obytes) ||
                     overlaps(uintptr_t(lse), lbytes, uintptr_t(lse_parts[i]), lbytes))))
            return fail(REGEN_ERR_INVALID_ARGUMENT, "an output overlaps an input part");
        mp.o[i] = static_cast<const uint16_t*>(o_parts[i]);
        mp.lse[i] = lse_parts[i];
    }
    if (lse && overlaps(uintptr_t(lse), lbytes, uintptr_t(o), obytes))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "lse overlaps o");
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return fail(REGEN_ERR_NO_DEVICE, "no HIP device is available");
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t threads = total * (head_dim / 8);
    const dim3 grid{unsigned((threads + 255) / 256), 1u, 1u};
    if (head_dim == 128)
        hipLaunchKernelGGL(regen::merge_parts_kernel<128>, grid, dim3(256), 0, st, mp, nparts,
                           (long long)total, static_cast<uint16_t*>(o), lse);
    else
        hipLaunchKernelGGL(regen::merge_parts_kernel<64>, grid, dim3(256), 0, st, mp, nparts,
                           (long long)total, static_cast<uint16_t*>(o), lse);
    e = hipGetLastError();
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    return REGEN_OK;
}

}  // extern "C"

namespace {

// dst [B][A][E] <- src [A][B][E], E = bytes per block (a multiple of 16).
regen_status block_transpose(const void* src, void* dst, int64_t A, int64_t B, int64_t E,
                             void* stream) {
    if (!src || !dst) return fail(REGEN_ERR_INVALID_ARGUMENT, "src and dst must be non-NULL");
    if (uintptr_t(src) % 16 != 0 || uintptr_t(dst) % 16 != 0)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "buffers must be 16-byte aligned");
    const int64_t bytes = A * B * E;
    if (overlaps(uintptr_t(src), uintptr_t(bytes), uintptr_t(dst), uintptr_t(bytes)))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "dst overlaps src");
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return fail(REGEN_ERR_NO_DEVICE, "no HIP device is available");
    }
    const int64_t n16 = bytes / 16;
    const dim3 grid{unsigned((n16 + 255) / 256), 1u, 1u};
    hipLaunchKernelGGL(regen::block_transpose_kernel, grid, dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), (long long)A, (long long)B, (long long)(E / 16));
    e = hipGetLastError();
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    return REGEN_OK;
}

regen_status ulysses_shape(int64_t tokens_local, int heads, int head_dim, int groups, int64_t* E) {
    if (tokens_local < 1 || heads < 1 || groups < 1 || head_dim < 1)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "tokens_local, heads, head_dim, groups must be >= 1");
    if (heads % groups != 0) return fail(REGEN_ERR_INVALID_ARGUMENT, "heads must be a multiple of groups");
    if ((int64_t(heads / groups) * head_dim * 2) % 16 != 0)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "(heads/groups) * head_dim * 2 must be a multiple of 16");
    if (tokens_local * heads * int64_t(head_dim) > (int64_t(1) << 40))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "tensor too large");
    *E = int64_t(heads / groups) * head_dim * 2;
    return REGEN_OK;
}

}  // namespace

extern "C" {

regen_status regen_ulysses_pack(const void* x, void* send, int64_t tokens_local, int heads,
                                int head_dim, int groups, void* stream) {
    g_last_error.clear();
    int64_t E = 0;
    regen_status s = ulysses_shape(tokens_local, heads, head_dim, groups, &E);
    if (s != REGEN_OK) return s;
    return block_transpose(x, send, tokens_local, groups, E, stream);
}

regen_status regen_ulysses_unpack(const void* recv, void* y, int64_t tokens_local, int heads,
                                  int head_dim, int groups, void* stream) {
    g_last_error.clear();
    int64_t E = 0;
    regen_status s = ulysses_shape(tokens_local, heads, head_dim, groups, &E);
    if (s != REGEN_OK) return s;
    return block_transpose(recv, y, groups, tokens_local, E, stream);
}

regen_status regen_clock_probe(int iters, int64_t* counters, double* wall_clock_khz, void* stream) {
    g_last_error.clear();
    if (iters < 1 || !counters || !wall_clock_khz)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "iters must be >= 1; counters and wall_clock_khz non-NULL");
    if (uintptr_t(counters) % 8 != 0) return fail(REGEN_ERR_INVALID_ARGUMENT, "counters must be 8-byte aligned");
    int dev = 0, cus = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute");
    *wall_clock_khz = double(khz);
    hipLaunchKernelGGL(regen::clock_probe_kernel, dim3(unsigned(std::max(1, cus))), dim3(512), 0,
                       static_cast<hipStream_t>(stream), reinterpret_cast<long long*>(counters), iters, 0.001f);
    e = hipGetLastError();
    if (e != hipSuccess) return fail_hip(e, "clock_probe_kernel launch");
    return REGEN_OK;
}

regen_status regen_attn_profile_read(regen_attn_t h, double* prep_ms, double* attn_ms,
                                     double* merge_ms, int64_t* calls) {
    g_last_error.clear();
    if (!h || !is_live(h)) return fail(REGEN_ERR_INVALID_ARGUMENT, "handle is NULL or not live");
    if (!(h->p.flags & REGEN_ATTN_PROFILE))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "handle was created without REGEN_ATTN_PROFILE");
    double tp = 0.0, ta = 0.0, tm = 0.0;
    int64_t n = 0;
    regen_status st = REGEN_OK;
    std::lock_guard<std::mutex> lk(h->mu);
    for (ProfRecord& r : h->prof_pending) {
        float a = 0.0f, b = 0.0f, c = 0.0f;
        hipError_t e = hipEventSynchronize(r.ev[3]);
        if (e == hipSuccess) e = hipEventElapsedTime(&a, r.ev[0], r.ev[1]);
        if (e == hipSuccess) e = hipEventElapsedTime(&b, r.ev[1], r.ev[2]);
        if (e == hipSuccess) e = hipEventElapsedTime(&c, r.ev[2], r.ev[3]);
        if (e != hipSuccess && st == REGEN_OK) st = fail_hip(e, "profile events");
        tp += a;
        ta += b;
        tm += c;
        ++n;
        h->prof_free.push_back(r);
    }
    h->prof_pending.clear();
    if (prep_ms) *prep_ms += tp;
    if (attn_ms) *attn_ms += ta;
    if (merge_ms) *merge_ms += tm;
    if (calls) *calls += n;
    return st;
}

regen_status regen_attn_destroy(regen_attn_t h) {
    g_last_error.clear();
    if (!h) return REGEN_OK;
    {
        std::lock_guard<std::mutex> lk(g_live_mu);
        if (!g_live.erase(h)) return fail(REGEN_ERR_INVALID_ARGUMENT, "handle is not live");
    }
    free_handle(h);
    return REGEN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Linear layers and the self-attention block
//   [Q | K | V] = X W_qkv^T,  O = attention(R Q, R K, V),  Y = O W_o^T.
// The projections run in gemm_nt_kernel; attention reads Q, K, V straight out
// of the fused projection output as strided token-major views and writes its
// output token-major, so nothing is copied between the three steps.
// ---------------------------------------------------------------------------
struct regen_block {
    regen_attn* attn;  // attention of the block (internal handle); its slots also
                       // hold the projection output and the attention output
    int N, hidden;
};

namespace {

std::mutex g_blocks_mu;
std::unordered_set<const void*> g_blocks;

bool block_live(const void* b) {
    std::lock_guard<std::mutex> lk(g_blocks_mu);
    return g_blocks.count(b) != 0;
}

void block_free(regen_block* b) {
    if (!b) return;
    if (b->attn) (void)regen_attn_destroy(b->attn);
    delete b;
}

// Resident workgroups per device of gemm_nt_kernel and gemm_nt256_kernel
// (CUs x workgroups per CU), queried once per device.
struct GemmSlots {
    int small, big;
};
std::mutex g_gemm_mu;
std::unordered_map<int, GemmSlots> g_gemm_slots;

regen_status gemm_slots(GemmSlots* slots) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_gemm_mu);
    auto it = g_gemm_slots.find(dev);
    if (it != g_gemm_slots.end()) {
        *slots = it->second;
        return REGEN_OK;
    }
    int cus = 0, per_cu = 0, per_cu_big = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return fail_hip(e, "hipDeviceGetAttribute");
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, regen::gemm_nt_kernel, 256, 0)) !=
            hipSuccess ||
        (e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_big, regen::gemm_nt256_kernel, 512, 0)) !=
            hipSuccess)
        return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    slots->small = std::max(1, cus) * std::max(1, per_cu);
    slots->big = std::max(1, cus) * std::max(1, per_cu_big);
    g_gemm_slots[dev] = *slots;
    return REGEN_OK;
}

regen_status gemm(const uint16_t* A, int lda, const uint16_t* B, int ldb, uint16_t* C, int ldc, int M,
                  int N, int K, hipStream_t st) {
    GemmSlots sl{1, 1};
    const regen_status s = gemm_slots(&sl);
    if (s != REGEN_OK) return s;
    // At least one full round of 256 x 256 tiles: the persistent kernel.
    const int64_t big_tiles = int64_t((M + regen::kGemmBig - 1) / regen::kGemmBig) *
                              ((N + regen::kGemmBig - 1) / regen::kGemmBig);
    if (big_tiles >= sl.big && big_tiles * 4 <= INT32_MAX) {
        hipLaunchKernelGGL(regen::gemm_nt256_kernel, dim3(unsigned(sl.big)), dim3(512), 0, st, A, lda, B,
                           ldb, C, ldc, M, N, K, int(big_tiles / sl.big));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail_hip(e, "gemm_nt256_kernel launch");
        return REGEN_OK;
    }
    const int slots = sl.small;
    const int64_t tiles = int64_t((M + regen::kGemmTile - 1) / regen::kGemmTile) *
                          ((N + regen::kGemmTile - 1) / regen::kGemmTile);
    // Quarter tiles for a short last round: only after at least one full
    // round, and only if the quarters still fit in one round.
    const int64_t full = tiles / slots * slots, rem = tiles - full;
    const int64_t nfull = (full > 0 && rem > 0 && rem * 4 <= slots) ? full : tiles;
    const int64_t blocks = nfull + (tiles - nfull) * 4;
    if (blocks > INT32_MAX) return fail(REGEN_ERR_INVALID_ARGUMENT, "too many output tiles");
    hipLaunchKernelGGL(regen::gemm_nt_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, A, lda, B, ldb,
                       C, ldc, M, N, K, int(nfull));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail_hip(e, "gemm_nt_kernel launch");
    return REGEN_OK;
}

}  // namespace

extern "C" {

regen_status regen_linear(const void* x, const void* w, void* y, int64_t rows, int in_features,
                          int out_features, void* stream) {
    g_last_error.clear();
    if (!x || !w || !y) return fail(REGEN_ERR_INVALID_ARGUMENT, "x, w, y must be non-NULL");
    if (rows < 1 || in_features < 1 || out_features < 1)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "rows, in_features, out_features must be >= 1");
    if (in_features % regen::kGemmBK != 0)
        return fail(REGEN_ERR_UNSUPPORTED, "in_features must be a multiple of 64");
    if (rows > (int64_t(1) << 30) || in_features > (1 << 20) || out_features > (1 << 20) ||
        rows * in_features * 2 >= (int64_t(1) << 32) ||
        int64_t(out_features) * in_features * 2 >= (int64_t(1) << 32))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "an operand exceeds 4 GiB");
    const uintptr_t ptrs[3] = {uintptr_t(x), uintptr_t(w), uintptr_t(y)};
    for (uintptr_t a : ptrs)
        if (a % 16 != 0) return fail(REGEN_ERR_INVALID_ARGUMENT, "x, w, y must be 16-byte aligned");
    const uintptr_t xb = uintptr_t(rows) * in_features * 2, wb = uintptr_t(out_features) * in_features * 2,
                    yb = uintptr_t(rows) * out_features * 2;
    if (overlaps(ptrs[2], yb, ptrs[0], xb) || overlaps(ptrs[2], yb, ptrs[1], wb))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "y overlaps x or w");
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return fail(REGEN_ERR_NO_DEVICE, "no HIP device is available");
    }
    return gemm(static_cast<const uint16_t*>(x), in_features, static_cast<const uint16_t*>(w),
                in_features, static_cast<uint16_t*>(y), out_features, int(rows), out_features,
                in_features, static_cast<hipStream_t>(stream));
}

regen_status regen_block_create(const regen_attn_desc* desc, regen_block_t* out) {
    g_last_error.clear();
    if (!out) return fail(REGEN_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    Problem p;
    regen_status s = resolve(desc, &p);
    if (s != REGEN_OK) return s;
    if (p.flags & (REGEN_ATTN_TOKEN_MAJOR | REGEN_ATTN_PROFILE))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "a block takes no layout or profiling flag");
    if (p.tokens * int64_t(p.heads) * p.head_dim * 3 * 2 >= (int64_t(1) << 32))
        return fail(REGEN_ERR_UNSUPPORTED, "the projection output would exceed 4 GiB");
    regen_block* b = new (std::nothrow) regen_block();
    if (!b) return fail(REGEN_ERR_OUT_OF_MEMORY, "host allocation of the block failed");
    s = regen_attn_create(desc, &b->attn);
    if (s != REGEN_OK) {
        delete b;
        return s;
    }
    b->N = int(p.tokens);
    b->hidden = p.heads * p.head_dim;
    const size_t H = size_t(b->hidden), N = size_t(b->N);
    hipError_t e = hipSuccess;
    for (Slot& sl : b->attn->slot) {
        if (e == hipSuccess) e = hipMalloc(&sl.qkv, N * 3 * H * 2);
        if (e == hipSuccess) e = hipMalloc(&sl.attn_out, N * H * 2);
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        block_free(b);
        return fail(e == hipErrorOutOfMemory ? REGEN_ERR_OUT_OF_MEMORY : REGEN_ERR_HIP,
                    std::string("device allocation failed: ") + hipGetErrorString(e));
    }
    {
        std::lock_guard<std::mutex> lk(g_blocks_mu);
        g_blocks.insert(b);
    }
    *out = b;
    return REGEN_OK;
}

regen_status regen_block_forward(regen_block_t b, const void* x, const void* w_qkv,
                                 const void* w_o, void* y, void* stream) {
    g_last_error.clear();
    if (!b || !block_live(b)) return fail(REGEN_ERR_INVALID_ARGUMENT, "block is NULL or not live");
    if (!x || !w_qkv || !w_o || !y)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "x, w_qkv, w_o, y must be non-NULL");
    const uintptr_t ptrs[4] = {uintptr_t(x), uintptr_t(w_qkv), uintptr_t(w_o), uintptr_t(y)};
    for (uintptr_t a : ptrs)
        if (a % 16 != 0) return fail(REGEN_ERR_INVALID_ARGUMENT, "x, w_qkv, w_o, y must be 16-byte aligned");
    const uintptr_t H = uintptr_t(b->hidden), N = uintptr_t(b->N);
    const uintptr_t xb = N * H * 2, wqb = H * 3 * H * 2, wob = H * H * 2;
    if (overlaps(ptrs[3], xb, ptrs[0], xb) || overlaps(ptrs[3], xb, ptrs[1], wqb) ||
        overlaps(ptrs[3], xb, ptrs[2], wob))
        return fail(REGEN_ERR_INVALID_ARGUMENT, "y overlaps x, w_qkv or w_o");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int Hd = b->hidden;
    regen_attn* h = b->attn;
    return with_slot(h, stream, [&](Slot* sl, ProfRecord* rec) {
        regen_status s = gemm(static_cast<const uint16_t*>(x), Hd, static_cast<const uint16_t*>(w_qkv), Hd,
                              sl->qkv, 3 * Hd, b->N, 3 * Hd, Hd, st);
        if (s != REGEN_OK) return s;
        const long long D = h->p.head_dim;
        const Strides sd{D, 3LL * Hd, D, 3LL * Hd, D, Hd};
        s = enqueue(handle_ctx(h, sl), sl->qkv, 0, b->N, sl->qkv + Hd, sl->qkv + 2 * Hd, 0, b->N,
                    sl->attn_out, nullptr, stream, false, sd, rec);
        if (s != REGEN_OK) return s;
        return gemm(sl->attn_out, Hd, static_cast<const uint16_t*>(w_o), Hd, static_cast<uint16_t*>(y), Hd,
                    b->N, Hd, Hd, st);
    });
}

regen_status regen_block_destroy(regen_block_t b) {
    g_last_error.clear();
    if (!b) return REGEN_OK;
    {
        std::lock_guard<std::mutex> lk(g_blocks_mu);
        if (!g_blocks.erase(b)) return fail(REGEN_ERR_INVALID_ARGUMENT, "block is not live");
    }
    block_free(b);
    return REGEN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The allocation-free forward (regen_attn_forward_noalloc): the kernels of
// regen_attn_forward, with the rotary table, the rotated K / transposed V and
// the split-tile partials in one file-scope device array. Its device address
// is looked up once per device (hipGetSymbolAddress) and only that address is
// handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[REGEN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
struct StaticDevice {
    unsigned char* ptr;  // device address of `scratch` on this device
    int slots[2];        // resident attention workgroups, head_dim 64 / 128
    int cross_slots[2];  // resident cross_attn_kernel workgroups, head_dim 64 / 128
    bool ready;
};
std::mutex g_static_mu;
StaticDevice g_static[kMaxDevices];

// Per-device set-up on first use, with the device current: the architecture
// check, the scratch array's device address, the resident workgroup counts.
regen_status static_device(int dev, StaticDevice* out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(REGEN_ERR_UNSUPPORTED, "device index above 63");
    std::lock_guard<std::mutex> lk(g_static_mu);
    StaticDevice& sd = g_static[dev];
    if (!sd.ready) {
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail_hip(e, "hipGetDeviceProperties");
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
            return fail(REGEN_ERR_UNSUPPORTED,
                        std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950");
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress of the static scratch");
        if (!ptr) return fail(REGEN_ERR_HIP, "hipGetSymbolAddress returned no address for the static scratch");
        int a64 = 1, c64 = 1, a128 = 1, c128 = 1;
        regen_status s = occupancy<64>(&a64, &c64);
        if (s == REGEN_OK) s = occupancy<128>(&a128, &c128);
        if (s != REGEN_OK) return s;
        const int cus = prop.multiProcessorCount;
        sd.ptr = static_cast<unsigned char*>(ptr);
        sd.slots[0] = a64 * cus;
        sd.slots[1] = a128 * cus;
        sd.cross_slots[0] = c64 * cus;
        sd.cross_slots[1] = c128 * cus;
        sd.ready = true;
    }
    *out = sd;
    return REGEN_OK;
}

}  // namespace

extern "C" {

regen_status regen_attn_forward_noalloc(const regen_attn_desc* desc, const void* q, const void* k,
                                        const void* v, void* o, void* stream) {
    g_last_error.clear();
    Problem p;
    regen_status s = resolve(desc, &p);
    if (s != REGEN_OK) return s;
    if (p.flags & REGEN_ATTN_PROFILE)
        return fail(REGEN_ERR_INVALID_ARGUMENT, "the allocation-free forward takes no profiling flag");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    StaticDevice sd{};
    s = static_device(dev, &sd);
    if (s != REGEN_OK) return s;
    const int hsel = p.head_dim == 128 ? 1 : 0;

    regen::RopeGeom geo;
    const int64_t entries = rope_geometry(p, &geo);
    const int P = int(std::min<int64_t>(sd.slots[hsel], p.units));
    // Scratch layout: table | Kr | Vt | partial O / l | partial (m, l) | piece
    // counter, each at a 256-byte boundary.
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t tab_b = up(size_t(entries) * sizeof(float2));
    const size_t half_ws = up(workspace_bytes(p) / 2);
    const size_t po_b = up(size_t(2) * P * kBM * p.head_dim * sizeof(uint16_t));
    const size_t pm_b = up(size_t(2) * P * kBM * 2 * sizeof(float));
    const size_t cnt_b = up(sizeof(int));
    const size_t need = tab_b + 2 * half_ws + po_b + pm_b + cnt_b;
    if (entries >= (int64_t(1) << 31) || need > REGEN_NOALLOC_SCRATCH_BYTES)
        return fail(REGEN_ERR_UNSUPPORTED,
                    "problem needs " + std::to_string(need) + " bytes of scratch; the allocation-free "
                    "forward holds " + std::to_string(size_t(REGEN_NOALLOC_SCRATCH_BYTES)) +
                    " (use regen_attn_create / regen_attn_forward)");
    s = check_call(p, q, 0, p.tokens, k, v, 0, p.tokens, o, nullptr, false);
    if (s != REGEN_OK) return s;
    unsigned char* base = sd.ptr;
    float2* tab = reinterpret_cast<float2*>(base);
    Ctx c{&p, &geo, tab, tab, P, sd.cross_slots[hsel],
          reinterpret_cast<uint16_t*>(base + tab_b),
          reinterpret_cast<uint16_t*>(base + tab_b + half_ws),
          reinterpret_cast<uint16_t*>(base + tab_b + 2 * half_ws),
          reinterpret_cast<float*>(base + tab_b + 2 * half_ws + po_b),
          reinterpret_cast<int*>(base + tab_b + 2 * half_ws + po_b + pm_b)};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(regen::rope_table_kernel, dim3(unsigned((entries + 255) / 256)), dim3(256), 0, st, tab,
                       geo, p.base, int(!(p.flags & REGEN_ATTN_NO_ROPE)), int(entries));
    e = hipGetLastError();
    if (e != hipSuccess) return fail_hip(e, "rope_table_kernel launch");
    return enqueue(c, q, 0, p.tokens, k, v, 0, p.tokens, o, nullptr, stream, false,
                   caller_strides(p, p.tokens, p.tokens), nullptr);
}

}  // extern "C"
