// api.cpp -- the C ABI: argument validation, schedule choice and launch.
//
// Every entry point validates everything it can on the host before touching
// the GPU, so argument errors are reported without a launch (and without a
// GPU).  Calls allocate nothing: the rank pointer tables are copied by value
// into the kernel arguments.  Calls are ordered on the caller's stream.
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/ar.h"
#include "ar_host.hpp"
#include "ar_kernels.hpp"

using namespace ar;

namespace {

const char *kDtypeName[] = {"fp32", "bf16", "fp16", "int32"};
const char *kOpName[] = {"sum", "prod", "min", "max", "avg"};
const char *kSchedName[] = {"AUTO", "RING", "TREE", "FUSED", "SPLIT", "DTREE"};
const char *kCollName[] = {"AllReduce", "ReduceScatter", "AllGather"};

bool valid_dtype(int d) { return d >= AR_FLOAT32 && d <= AR_INT32; }
bool valid_op(int o) { return o >= AR_SUM && o <= AR_AVG; }
bool valid_sched(int s) { return s >= AR_SCHED_AUTO && s <= AR_SCHED_DTREE; }

// Environment settings are read once, in initialisers of function-local
// statics (thread-safe: concurrent callers of the C ABI see one value).
bool debug_enabled() {
    static const bool v = [] {
        const char *e = getenv("AR_DEBUG");
        return e && *e && strcmp(e, "0") != 0;
    }();
    return v;
}

ar_sched_t forced_schedule() {
    const char *e = getenv("AR_SCHEDULE");
    if (!e) return AR_SCHED_AUTO;
    if (!strcmp(e, "ring")) return AR_SCHED_RING;
    if (!strcmp(e, "tree")) return AR_SCHED_TREE;
    if (!strcmp(e, "fused")) return AR_SCHED_FUSED;
    if (!strcmp(e, "split")) return AR_SCHED_SPLIT;
    if (!strcmp(e, "dtree")) return AR_SCHED_DTREE;
    return AR_SCHED_AUTO;
}

// Compute units of each device, queried once.
std::atomic<int> g_cus[64];

ar_status_t device_cus(int *cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return AR_ERR_HIP;
    if (dev < 0 || dev >= 64) return AR_ERR_HIP;
    int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || v <= 0) {
            if (debug_enabled()) fprintf(stderr, "[ar] device query failed: %d\n", (int)e);
            return AR_ERR_HIP;
        }
        g_cus[dev].store(v, std::memory_order_relaxed);
    }
    *cus = v;
    return AR_OK;
}


// Dynamic LDS (bytes) a fused workgroup reserves to cap how many one-wave
// workgroups are resident per CU (LDS is 160 KB per CU on gfx950).  Measured
// on MI355X with gradient-like data: every collective wants fewer resident
// workgroups the more ranks it streams (the per-rank-count tables in
// ar_kernels.hpp; past 16 ranks the all-reduce's wide kernel runs uncapped,
// the all-gather reserves 64 KB and the reduce-scatter 48 KB).  AR_FUSED_LDS_KB
// overrides all of them.
int fused_lds_bytes(ar_coll_t coll, int n) {
    const char *e = getenv("AR_FUSED_LDS_KB");                  // read per call: a tuning knob
    const long env = (e && *e) ? (atol(e) > 64 ? 64 : atol(e)) : -1;
    if (env >= 0) return (int)env * 1024;
    switch (coll) {
    case AR_COLL_ALLREDUCE: return (n >= 0 && n <= 16 ? kFusedLdsAllReduceByN[n] : kFusedLdsAllReduceKB) * 1024;
    case AR_COLL_ALL_GATHER: return (n >= 0 && n <= 16 ? kFusedLdsAllGatherByN[n] : kFusedLdsAllGatherKB) * 1024;
    default: return (n >= 0 && n <= 16 ? kFusedLdsReduceScatterByN[n] : kFusedLdsReduceScatterKB) * 1024;
    }
}

// The all-gather's cap for ``input`` bytes of pieces in all.  The table's caps
// (three or so one-wave workgroups per CU from 8 ranks on) were measured with
// the pieces resident in the 256 MB Infinity Cache, where back-to-back calls
// find them and the stores alone set the pace.  Past the cache every piece
// streams from HBM and those caps leave too few loads in flight: measured on
// MI355X with 512 MB-2 GB of pieces (fp32, % of peak, table cap -> 36 KB),
// 8 ranks 63-66 -> 70-73, 16 ranks 54-60 -> 75-79, 17 ranks 54 -> 68-75, 24
// ranks 62-64 -> 64-71; the ring ran 63-71, 64, 37 and 27.  At 72 ranks the
// caps measured level (62.7 against 63.7-64.2 at 64 KB), so past 32 ranks the
// table's cap stays.
int gather_lds_bytes(int n, double input) {
    const int lds = fused_lds_bytes(AR_COLL_ALL_GATHER, n);
    if (getenv("AR_FUSED_LDS_KB") || input <= kCacheBytes || n > 32) return lds;
    return lds < kGatherStreamLds ? lds : kGatherStreamLds;
}

// AR_TREE_STAGED=1 sends the n <= 16 tree schedules through the any-n
// kernels (as for n > 16: the streaming walk, or the LDS-staged kernels under
// AR_TREE_STREAM=0) instead of the register-evaluated ones; all give the same
// bits.  Read on every call (a getenv is far below a launch's cost),
// so one process can compare the kernels.
bool tree_staged() {
    const char *e = getenv("AR_TREE_STAGED");
    return e && *e == '1';
}

// AR_DWORD_VECTORS=0 sends all-reduces, reduce-scatters and all-gathers at
// mixed 16-byte phases with 4-byte-aligned pointers back to the element-wise
// kernels (same bits) instead of the vector kernels on the callers' pointers;
// read on every call.
bool dword_vectors() {
    const char *e = getenv("AR_DWORD_VECTORS");
    return !(e && *e == '0');
}

// Whether a fused all-reduce past 16 ranks runs as the reduce-scatter half
// (the phased kernel's layout over the all-reduce's own chunks, each finished
// chunk stored to its owner) then the all-gather half (each chunk copied from
// its owner to the other ranks), instead of the wide one-pass kernel: S more
// bytes than the 2*n*S of one pass, the same hop order and bits.  Measured on
// MI355X, 25 MB per rank in place, % of peak (wide -> halves; split on the same
// box): fp32 n = 24 62.0 -> 63.5 (70.1), 72 60.7 -> 66.6 (67.3), 128 61.2 ->
// 68.9 (65.2); bf16 n = 33 60.1 -> 67.4 (68.4), 72 60.0 -> 70.8 (66.3).
// AR_AR_HALVES=0 keeps the wide kernel (read on every call).
bool allreduce_halves() {
    const char *e = getenv("AR_AR_HALVES");
    return !(e && *e == '0');
}

// Whether an aligned fused reduce-scatter past 16 ranks takes the phased
// kernel's layout (its word-aligned chain on aligned slices: four-wavefront
// workgroups on consecutive tiles, one vector per lane, ranks in batches of 8)
// instead of the any-n fused kernel's (one-wavefront workgroups, two vectors
// per lane, batches of 8 ranks per vector pair).  Same hop order, same bits.
// Measured on MI355X, % of peak (fused -> phased): bf16 n = 17 56.6 -> 70.7,
// 24 65.3 -> 79.1, 32 70.3 -> 78.3, 72 67.8 -> 76.5, 100 72.9 -> 76.8; fp32
// n = 17 66.7 -> 72.9, 20 71.0 -> 76.1, 33 71.9 -> 74.1, but 24 76.8 -> 75.7,
// 40 78.2 -> 75.8, 48 79.9 -> 77.5, 65 74.8 -> 71.7, 72 77.6 -> 75.7, 100
// 79.0 -> 77.5, 128 80.3 -> 78.8; up to 16 ranks the fused kernels lead or
// tie.  AR_RS_PHASED=0|1 overrides (read on every call).
bool rs_through_phased(int n, ar_dtype_t dt) {
    const char *e = getenv("AR_RS_PHASED");
    if (e && (*e == '0' || *e == '1')) return *e == '1';
    if (n <= 16) return false;
    if (dt == AR_BFLOAT16 || dt == AR_FLOAT16) return true;
    return n <= 35 && n % 8 != 0;
}

// Dynamic LDS reservation (bytes) of the ring / tree workgroups; the
// AR_RING_LDS_KB variable overrides the default.
int env_kb(const char *name, int dflt) {
    const char *e = getenv(name);
    long kb = (e && *e) ? atol(e) : dflt;
    if (kb < 0) return -1;
    return (int)(kb > 64 ? 64 : kb) * 1024;
}
int ring_lds_bytes(ar_coll_t coll, int n) {
    static const int v = env_kb("AR_RING_LDS_KB", -1);
    if (v >= 0) return v;
    if (coll == AR_COLL_ALLREDUCE) return (n >= 0 && n <= 16 ? kRingLdsAllReduceByN[n] : 0) * 1024;
    return (coll == AR_COLL_ALL_GATHER ? kRingLdsAllGatherKB : kRingLdsKB) * 1024;
}

// Window width (16-byte vectors per rank) for the LDS-staged schedules:
// n * W items of one workgroup, at most kThreads * kItemsPerThread.
int lds_window(int n) {
    int w = (n <= 32) ? (kThreads * 2) / n : (kThreads * kItemsPerThread) / n;
    return w < 1 ? 1 : w;
}

// Window width of the LDS-staged trees: a multiple of 8 vectors, so that a
// window covers whole 128-byte lines of every rank buffer (a width of 14
// vectors at 72 ranks read and wrote partial lines), with n * W at most
// kThreads * kItemsPerThread items.
int tree_window(int n) {
    const int w = (kThreads * kItemsPerThread) / (8 * n) * 8;
    return w < 8 ? 8 : w;
}

// The 16-byte phase (address mod 16) shared by n pointers, or -1.
int one_phase(const void *const *p, int n) {
    const int ph = (int)((uintptr_t)p[0] & 15);
    for (int r = 1; r < n; ++r)
        if ((int)((uintptr_t)p[r] & 15) != ph) return -1;
    return ph;
}

// The 16-byte phase (address mod 16) shared by all 2n pointers, or -1.
int common_phase(const void *const *a, const void *const *b, int n) {
    const int ph = (int)((uintptr_t)a[0] & 15);
    for (int r = 0; r < n; ++r)
        if ((int)((uintptr_t)a[r] & 15) != ph || (int)((uintptr_t)b[r] & 15) != ph) return -1;
    return ph;
}

bool null_entry(const void *const *p, int n) {
    for (int r = 0; r < n; ++r)
        if (!p[r]) return true;
    return false;
}

bool misaligned(const void *const *p, int n, size_t align) {
    for (int r = 0; r < n; ++r)
        if ((uintptr_t)p[r] % align) return true;
    return false;
}

bool all16(const void *const *a, const void *const *b, int n) {
    for (int r = 0; r < n; ++r)
        if (((uintptr_t)a[r] | (uintptr_t)b[r]) & 15u) return false;
    return true;
}

// recv range r may coincide with its own in-place position (``inplace[r]``
// set: the layout the header allows for rank r) and must not otherwise
// overlap any send range or any other recv range; send ranges may overlap
// each other.  Every recv range is a writable span and every send range a
// read-only span, except that for an allowed (send r, recv r) pair only the
// parts of send r outside recv r are emitted (read-only), so the pair does not
// conflict with itself.  After sorting by start, a span conflicts iff it
// starts before the end of an earlier writable span, or is writable and starts
// before the end of any earlier span.  O(n log n) for up to 3n spans.
struct Span {
    uintptr_t lo, hi;
    bool writable;
};

ar_status_t check_overlap(const void *const *send, size_t slen, void *const *recv, size_t rlen, int n,
                          const uintptr_t *inplace) {
    Span sp[3 * AR_MAX_RANKS];
    int m = 0;
    for (int r = 0; r < n; ++r) {
        const uintptr_t s0 = (uintptr_t)send[r], s1 = s0 + slen;
        const uintptr_t d0 = (uintptr_t)recv[r], d1 = d0 + rlen;
        sp[m++] = {d0, d1, true};
        if (!inplace[r]) {
            sp[m++] = {s0, s1, false};
            continue;
        }
        if (s0 < d0) sp[m++] = {s0, s1 < d0 ? s1 : d0, false};      // send r below recv r
        if (s1 > d1) sp[m++] = {s0 > d1 ? s0 : d1, s1, false};      // send r above recv r
    }
    std::sort(sp, sp + m, [](const Span &a, const Span &b) { return a.lo < b.lo; });
    uintptr_t end_all = 0, end_w = 0;
    for (int i = 0; i < m; ++i) {
        if (i > 0 && (sp[i].lo < end_w || (sp[i].writable && sp[i].lo < end_all))) return AR_ERR_INVALID_ARG;
        if (sp[i].hi > end_all) end_all = sp[i].hi;
        if (sp[i].writable && sp[i].hi > end_w) end_w = sp[i].hi;
    }
    return AR_OK;
}

void log_plan(ar_coll_t coll, size_t bytes_per_rank, int n, int dtype, int op, const ar_plan_t &p, ar_sched_t used,
              bool forced) {
    if (!debug_enabled()) return;
    fprintf(stderr,
            "[ar] %s: %zu Bytes x n=%d %s %s -> %s%s (predicted us: ring %.2f tree %.2f fused %.2f split %.2f "
            "dtree %.2f; calib %s)\n",
            kCollName[coll], bytes_per_rank, n, kDtypeName[dtype], kOpName[op], kSchedName[used],
            forced ? " (forced)" : "", p.predicted_us[AR_SCHED_RING], p.predicted_us[AR_SCHED_TREE],
            p.predicted_us[AR_SCHED_FUSED], p.predicted_us[AR_SCHED_SPLIT], p.predicted_us[AR_SCHED_DTREE],
            calib_source());
}

// Resolve AR_SCHED_AUTO (and the AR_SCHEDULE override) into a legal schedule;
// ``allowed`` further restricts the legal set (numerics some schedules lack).
ar_status_t choose(ar_coll_t coll, size_t count, ar_dtype_t dtype, ar_op_t op, int n, ar_sched_t sched,
                   ar_sched_t *out, size_t bytes_per_rank, unsigned allowed = ~0u) {
    ar_plan_t p;
    ar_status_t st = make_plan(coll, count, dtype, op, n, &p);
    if (st != AR_OK) return st;
    if ((p.legal_mask & allowed) != p.legal_mask) {             // re-pick among what is left
        p.legal_mask &= allowed;
        double best = 0;
        bool have = false;
        for (int s = AR_SCHED_RING; s <= AR_SCHED_DTREE; ++s) {
            if (!(p.legal_mask & (1u << s))) continue;
            if (!have || p.predicted_us[s] < best) {
                best = p.predicted_us[s];
                p.chosen = (ar_sched_t)s;
                have = true;
            }
        }
    }
    bool forced = sched != AR_SCHED_AUTO;
    if (!forced) {
        ar_sched_t env = forced_schedule();
        if (env != AR_SCHED_AUTO && (p.legal_mask & (1u << env))) {
            sched = env;
            forced = true;
        }
    }
    if (sched == AR_SCHED_AUTO) sched = p.chosen;
    if (!(p.legal_mask & (1u << sched))) return AR_ERR_UNSUPPORTED;
    log_plan(coll, bytes_per_rank, n, dtype, op, p, sched, forced);
    *out = sched;
    return AR_OK;
}

ar_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return AR_OK;
    if (debug_enabled()) fprintf(stderr, "[ar] HIP error %d: %s\n", (int)e, hipGetErrorString(e));
    return AR_ERR_HIP;
}

void fill_table(RankTable &t, const void *const *send, void *const *recv, int n) {
    memset(&t, 0, sizeof t);
    for (int r = 0; r < n; ++r) {
        t.src[r] = send[r];
        t.dst[r] = recv[r];
    }
}

ar_status_t common_checks(const void *const *send, void *const *recv, int dtype, int op, int n, int sched) {
    if (n < 1 || n > AR_MAX_RANKS || !send || !recv) return AR_ERR_INVALID_ARG;
    if (!valid_dtype(dtype) || !valid_op(op) || !valid_sched(sched)) return AR_ERR_INVALID_ARG;
    return AR_OK;
}

// The numerics of a call in the geometry: the float avg pre-scale s (1/n, or
// 1/p for the split route with p = 2^e, e the least with 4^e >= n), the split
// route's post-divisor n/p, and fp32 partials for bf16 / fp16.  Returns the
// schedules that support them (fp32 partials: the fused pass only, where the
// partials never leave registers).
ar_status_t apply_numerics(const ar_numerics_t *num, int dtype, int op, int n, Geometry &g, unsigned *allowed) {
    *allowed = ~0u;
    g.s = (float)(1.0 / (double)n);
    g.post_div = 0.0f;
    g.acc32 = 0;
    if (!num) return AR_OK;
    if ((num->acc != AR_ACC_STORAGE && num->acc != AR_ACC_FP32) ||
        (num->avg != AR_AVG_PRESCALE && num->avg != AR_AVG_SPLIT))
        return AR_ERR_INVALID_ARG;
    const bool is_float = dtype != AR_INT32;
    if (num->avg == AR_AVG_SPLIT && is_float && op == AR_AVG) {
        int p = 1;
        while (p * p < n) p *= 2;
        g.s = (float)(1.0 / (double)p);
        g.post_div = (float)((double)n / (double)p);           // exact: n <= 128, p a power of two
    }
    if (num->acc == AR_ACC_FP32 && (dtype == AR_BFLOAT16 || dtype == AR_FLOAT16)) {
        g.acc32 = 1;
        *allowed = 1u << AR_SCHED_FUSED;
    }
    return AR_OK;
}

}  // namespace

// Workgroups for a persistent launch over ``units`` independent work units:
// per_cu per compute unit (AR_GRID overrides), at most ``units``.
int ar::grid_for(long long units, int cus, int per_cu) {
    const char *e = getenv("AR_GRID");
    long long g = (e && atoll(e) > 0) ? atoll(e) : (long long)cus * per_cu;
    if (g > units) g = units;
    return (int)(g < 1 ? 1 : g);
}

extern "C" {

const char *ar_status_string(ar_status_t s) {
    switch (s) {
    case AR_OK: return "AR_OK";
    case AR_ERR_INVALID_ARG: return "AR_ERR_INVALID_ARG: invalid argument";
    case AR_ERR_UNSUPPORTED: return "AR_ERR_UNSUPPORTED: schedule not legal for this collective";
    case AR_ERR_ALIGNMENT: return "AR_ERR_ALIGNMENT: buffer not aligned to its element size";
    case AR_ERR_HIP: return "AR_ERR_HIP: HIP runtime error";
    default: return "unknown ar_status_t";
    }
}

int ar_tree_parent(int n, int v) { return (n >= 1 && n <= AR_MAX_RANKS) ? tree_parent(n, v) : -1; }

int ar_dtree_parent(int n, int which, int v) {
    return (n >= 1 && n <= AR_MAX_RANKS && (which == 0 || which == 1)) ? dtree_parent(n, which, v) : -1;
}

ar_status_t ar_plan(ar_coll_t coll, size_t count, ar_dtype_t dtype, ar_op_t op, int n, ar_plan_t *out) {
    if (!out || n < 1 || n > AR_MAX_RANKS || !valid_dtype(dtype) || !valid_op(op) || (int)coll < 0 ||
        (int)coll > AR_COLL_ALL_GATHER)
        return AR_ERR_INVALID_ARG;
    return make_plan(coll, count, dtype, op, n, out);
}

ar_status_t ar_allreduce(const void *const *sendbufs, void *const *recvbufs, size_t count, ar_dtype_t dtype,
                         ar_op_t op, int n, ar_sched_t sched, hipStream_t stream) {
    return ar_allreduce_ex(sendbufs, recvbufs, count, dtype, op, n, sched, nullptr, stream);
}

ar_status_t ar_allreduce_ex(const void *const *sendbufs, void *const *recvbufs, size_t count, ar_dtype_t dtype,
                            ar_op_t op, int n, ar_sched_t sched, const ar_numerics_t *numerics, hipStream_t stream) {
    ar_status_t st = common_checks(sendbufs, recvbufs, dtype, op, n, sched);
    if (st != AR_OK) return st;
    if (count == 0) return AR_OK;
    if (null_entry(sendbufs, n) || null_entry((const void *const *)recvbufs, n)) return AR_ERR_INVALID_ARG;
    const size_t e = elem_size(dtype);
    if (count > (SIZE_MAX / 2) / e) return AR_ERR_INVALID_ARG;
    if (misaligned(sendbufs, n, e) || misaligned((const void *const *)recvbufs, n, e)) return AR_ERR_ALIGNMENT;
    uintptr_t inplace[AR_MAX_RANKS];
    for (int r = 0; r < n; ++r) inplace[r] = (recvbufs[r] == sendbufs[r]) ? 1 : 0;
    st = check_overlap(sendbufs, count * e, recvbufs, count * e, n, inplace);
    if (st != AR_OK) return st;
    Geometry g;
    memset(&g, 0, sizeof g);
    unsigned allowed;
    st = apply_numerics(numerics, dtype, op, n, g, &allowed);
    if (st != AR_OK) return st;
    ar_sched_t use;
    st = choose(AR_COLL_ALLREDUCE, count, dtype, op, n, sched, &use, count * e, allowed);
    if (st != AR_OK) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != AR_OK) return st;

    RankTable t;
    fill_table(t, sendbufs, recvbufs, n);
    const long long lanes = 16 / (long long)e;
    g.n = n;
    g.V = ((long long)count + lanes - 1) / lanes;
    g.Vfull = (long long)count / lanes;
    g.q = g.V / n;
    g.rem = (int)(g.V % n);
    g.ref = (long long)((uintptr_t)recvbufs[0] >> 4);          // fused / split tiles follow rank 0's output
    TreeShape tree, tree2;
    if (use == AR_SCHED_TREE || use == AR_SCHED_DTREE) tree_build(n, tree, 0);
    if (use == AR_SCHED_DTREE) tree_build(n, tree2, 1);
    g.split = g.V / 2;                                          // dtree: vectors up the first tree (<= Vfull)

    auto elem = [&](long long e_begin) {
        if (use == AR_SCHED_TREE) return launch_elem_tree_allreduce(dtype, op, t, tree, g, e_begin, (long long)count, stream);
        if (use == AR_SCHED_DTREE) {                                // two element ranges, one per tree
            const long long cut = g.split * lanes;
            hipError_t e1 = launch_elem_tree_allreduce(dtype, op, t, tree, g, e_begin, cut > e_begin ? cut : e_begin, stream);
            if (e1 != hipSuccess) return e1;
            return launch_elem_tree_allreduce(dtype, op, t, tree2, g, cut > e_begin ? cut : e_begin, (long long)count, stream);
        }
        if (use == AR_SCHED_SPLIT) return launch_elem_split_allreduce(dtype, op, t, g, e_begin, (long long)count, stream);
        return launch_elem_ring_allreduce(dtype, op, t, g, e_begin, (long long)count, stream);
    };
    g.split2 = g.split;

    // The schedule's vector kernels over frame vectors [0, g.Vfull) of the pointers in ``tv``.
    auto vectors = [&](const RankTable &tv) -> ar_status_t {
        hipError_t h = hipSuccess;
        if (g.Vfull <= 0) return AR_OK;
        if (use == AR_SCHED_SPLIT) {
            if ((g.Vfull + kFusedTile - 1) / kFusedTile > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;   // grid x limit
            h = launch_split_allreduce(dtype, op, tv, g, stream);
        } else if (use == AR_SCHED_FUSED) {
            const long long maxlen = (g.V + n - 1) / n;                       // longest chunk, in vectors
            g.windows = aligned_tiles(maxlen, kFusedTile);
            if (g.windows > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;   // grid x limit
            if (n > 16 && allreduce_halves())
                h = launch_allreduce_halves(dtype, op, tv, g, fused_lds_bytes(AR_COLL_REDUCE_SCATTER, n),
                                            gather_lds_bytes(n, (double)count * (double)e), stream);
            else
                h = launch_fused_allreduce(dtype, op, tv, g, fused_lds_bytes(AR_COLL_ALLREDUCE, n), stream);
        } else if (use == AR_SCHED_RING) {
            g.W = lds_window(n);
            const long long maxlen = (g.V + n - 1) / n;
            g.windows = (maxlen + g.W - 1) / g.W;
            h = launch_ring_allreduce(dtype, op, tv, g, grid_for(g.windows, cus, 4), ring_lds_bytes(AR_COLL_ALLREDUCE, n), stream);
        } else if (n >= 2 && n <= 16 && !tree_staged()) {               // tree / dtree, in registers
            if (aligned_tiles(g.Vfull, kFusedTile) > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;   // grid x limit
            h = launch_tree_reg_allreduce(use == AR_SCHED_DTREE, dtype, op, tv, g,
                                          fused_lds_bytes(AR_COLL_ALLREDUCE, n), stream);
        } else if (use == AR_SCHED_DTREE) {
            g.W = tree_window(n);
            h = launch_dtree_allreduce(dtype, op, tv, tree, tree2, g, cus, stream);
        } else {
            g.W = tree_window(n);
            h = launch_tree_allreduce(dtype, op, tv, tree, g, cus, stream);
        }
        return hip_status(h);
    };

    if (all16(sendbufs, (const void *const *)recvbufs, n)) {
        st = vectors(t);
        if (st != AR_OK) return st;
        if (g.Vfull * lanes < (long long)count) return hip_status(elem(g.Vfull * lanes));   // tail: count mod lanes
        return AR_OK;
    }

    // Buffers off 16-byte alignment.  When all 2n pointers sit at the same
    // 16-byte phase, the vectors run in the frame that starts at the first
    // 16-byte boundary (``head`` elements in), with the chunks and the double
    // tree's split still those of element index 0; the element-wise kernels
    // take exactly the rest: each chunk's first ``head`` elements and the frame
    // vector across its end (ring order), the head, the vector across the
    // double tree's split and the tail (tree orders).  Otherwise, or for the
    // LDS-staged ring past 16 ranks, 4-byte elements in ring order take the
    // fused vector kernels on the callers' pointers and everything else goes
    // element-wise.
    const int ph = common_phase(sendbufs, (const void *const *)recvbufs, n);
    const long long head = ph > 0 ? (long long)((16 - ph) / (int)e) : 0;
    const bool frame = ph > 0 && (long long)count > head && !(use == AR_SCHED_RING && n > 16);
    if (!frame && !misaligned(sendbufs, n, 4) && !misaligned((const void *const *)recvbufs, n, 4) &&
        (use == AR_SCHED_FUSED || use == AR_SCHED_RING) && dword_vectors()) {
        // Mixed phases (or the ring past 16 ranks) with every pointer 4-byte aligned (always so for 4-byte
        // elements): that is all the fused kernels' 16-byte accesses need, so they run on the callers'
        // pointers, vector v of every buffer at byte 16*v, in the ring's hop order (the ring schedule's
        // bits), and the element-wise kernel takes the count mod lanes tail.
        use = AR_SCHED_FUSED;
        st = vectors(t);
        if (st != AR_OK) return st;
        if (g.Vfull * lanes < (long long)count) return hip_status(elem(g.Vfull * lanes));
        return AR_OK;
    }
    if (!frame) return hip_status(elem(0));
    RankTable tv = t;
    for (int r = 0; r < n; ++r) {
        tv.src[r] = (const char *)sendbufs[r] + head * (long long)e;
        tv.dst[r] = (char *)recvbufs[r] + head * (long long)e;
    }
    const long long S = g.split;                                // the double tree's split, in element-index vectors
    g.shift = 1;
    g.Vfull = ((long long)count - head) / lanes;
    g.ref = (long long)((uintptr_t)tv.dst[0] >> 4);
    g.split = S >= 1 ? (S - 1 < g.Vfull ? S - 1 : g.Vfull) : 0;  // frame vectors wholly below element lanes*S
    g.split2 = S < g.Vfull ? S : g.Vfull;                       // ... and wholly at or above it
    st = vectors(tv);
    if (st != AR_OK) return st;
    if (use == AR_SCHED_FUSED || use == AR_SCHED_RING)
        return hip_status(launch_elem_ring_gaps(dtype, op, t, g, head, (long long)count, stream));
    const long long end = head + lanes * g.Vfull;               // element ranges the vectors left
    const long long ranges[3][2] = {{0, head},
                                    {head + lanes * g.split, use == AR_SCHED_DTREE ? head + lanes * g.split2
                                                                                   : head + lanes * g.split},
                                    {end, (long long)count}};
    for (const auto &rg : ranges) {
        if (rg[1] <= rg[0]) continue;
        hipError_t h;
        if (use == AR_SCHED_SPLIT) {
            h = launch_elem_split_allreduce(dtype, op, t, g, rg[0], rg[1], stream);
        } else if (use == AR_SCHED_TREE) {
            h = launch_elem_tree_allreduce(dtype, op, t, tree, g, rg[0], rg[1], stream);
        } else {                                                // dtree: element index lanes*S splits the trees
            const long long cut = lanes * S;
            const long long m = cut < rg[0] ? rg[0] : (cut > rg[1] ? rg[1] : cut);
            h = launch_elem_tree_allreduce(dtype, op, t, tree, g, rg[0], m, stream);
            if (h == hipSuccess) h = launch_elem_tree_allreduce(dtype, op, t, tree2, g, m, rg[1], stream);
        }
        if (h != hipSuccess) return hip_status(h);
    }
    return AR_OK;
}

ar_status_t ar_reduce_scatter(const void *const *sendbufs, void *const *recvbufs, size_t recvcount,
                              ar_dtype_t dtype, ar_op_t op, int n, ar_sched_t sched, hipStream_t stream) {
    return ar_reduce_scatter_ex(sendbufs, recvbufs, recvcount, dtype, op, n, sched, nullptr, stream);
}

ar_status_t ar_reduce_scatter_ex(const void *const *sendbufs, void *const *recvbufs, size_t recvcount,
                                 ar_dtype_t dtype, ar_op_t op, int n, ar_sched_t sched,
                                 const ar_numerics_t *numerics, hipStream_t stream) {
    ar_status_t st = common_checks(sendbufs, recvbufs, dtype, op, n, sched);
    if (st != AR_OK) return st;
    if (recvcount == 0) return AR_OK;
    if (null_entry(sendbufs, n) || null_entry((const void *const *)recvbufs, n)) return AR_ERR_INVALID_ARG;
    const size_t e = elem_size(dtype);
    if (recvcount > (SIZE_MAX / 2) / e / (size_t)n) return AR_ERR_INVALID_ARG;
    if (misaligned(sendbufs, n, e) || misaligned((const void *const *)recvbufs, n, e)) return AR_ERR_ALIGNMENT;
    uintptr_t inplace[AR_MAX_RANKS];
    for (int r = 0; r < n; ++r)
        inplace[r] = ((uintptr_t)recvbufs[r] == (uintptr_t)sendbufs[r] + (uintptr_t)r * recvcount * e) ? 1 : 0;
    st = check_overlap(sendbufs, (size_t)n * recvcount * e, recvbufs, recvcount * e, n, inplace);
    if (st != AR_OK) return st;
    Geometry g;
    memset(&g, 0, sizeof g);
    unsigned allowed;
    st = apply_numerics(numerics, dtype, op, n, g, &allowed);
    if (st != AR_OK) return st;
    ar_sched_t use;
    st = choose(AR_COLL_REDUCE_SCATTER, recvcount, dtype, op, n, sched, &use, (size_t)n * recvcount * e, allowed);
    if (st != AR_OK) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != AR_OK) return st;

    RankTable t;
    fill_table(t, sendbufs, recvbufs, n);
    g.n = n;
    const bool vec = all16(sendbufs, (const void *const *)recvbufs, n) && (recvcount * e) % 16 == 0;
    if (!vec) {
        // Slices that are not whole 16-byte vectors, or buffers off 16-byte alignment.  With every input at
        // one 16-byte phase and every output at one phase, the phased pass (any schedule: the ring computes
        // the same hop order) writes every whole vector of the output frame that starts at the outputs' first
        // 16-byte boundary, reading the inputs through aligned pairs of vectors; the element-wise kernel
        // takes each output's first and last few elements.  At mixed phases with every pointer 4-byte aligned
        // (always so for 4-byte elements) the phased pass's word-aligned loads run on the callers' pointers
        // (output vector o of every slice at byte 16*o, every access 4-byte aligned, which is all a 16-byte
        // access needs, and inside the words holding the lane's own bytes) and the element-wise kernel takes
        // each slice's last R mod lanes elements; other alignments go element-wise.
        const long long R = (long long)recvcount, Rb = R * (long long)e;
        const int ps = one_phase(sendbufs, n), pr = one_phase((const void *const *)recvbufs, n);
        const long long head = pr > 0 ? (long long)((16 - pr) / (int)e) : 0;
        if (ps < 0 || pr < 0 || head >= R) {
            if (misaligned(sendbufs, n, 4) || misaligned((const void *const *)recvbufs, n, 4) || !dword_vectors())
                return hip_status(launch_elem_reduce_scatter(dtype, op, t, g, R, 0, 0, stream));
            g.slice_bytes = Rb;
            g.Rv = Rb / 16;
            g.phased_words = 2;                                     // the word-aligned loads only
            if (aligned_tiles(g.Rv, kFusedTile) > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;   // grid x limit
            const hipError_t h = launch_fused_reduce_scatter_phased(dtype, op, t, g,
                                                                    fused_lds_bytes(AR_COLL_REDUCE_SCATTER, n), stream);
            if (h != hipSuccess) return hip_status(h);
            return hip_status(launch_elem_reduce_scatter(dtype, op, t, g, R, 0, g.Rv * (long long)(16 / e), stream));
        }
        g.slice_bytes = Rb;
        g.out_off = head * (long long)e;
        g.in_off = ps + g.out_off;
        g.Rv = (Rb - g.out_off) / 16;
        g.last_off = ((ps + (long long)n * Rb - 1) >> 4) << 4;
        if (aligned_tiles(g.Rv, kFusedTile) > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;   // grid x limit
        RankTable tp = t;
        for (int r = 0; r < n; ++r) {
            tp.src[r] = (const char *)sendbufs[r] - ps;
            tp.dst[r] = (char *)recvbufs[r] + g.out_off;
        }
        const hipError_t h = launch_fused_reduce_scatter_phased(dtype, op, tp, g,
                                                                fused_lds_bytes(AR_COLL_REDUCE_SCATTER, n), stream);
        if (h != hipSuccess) return hip_status(h);
        return hip_status(launch_elem_reduce_scatter(dtype, op, t, g, R, head, head + g.Rv * (long long)(16 / e), stream));
    }
    g.Rv = (long long)(recvcount * e / 16);
    g.ref = (long long)((uintptr_t)sendbufs[0] >> 4);          // fused tiles follow the input slices' alignment
    if (use == AR_SCHED_FUSED) {
        if (aligned_tiles(g.Rv, kFusedTile) > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;   // grid x limit
        if (rs_through_phased(n, dtype)) {
            g.slice_bytes = (long long)recvcount * (long long)e;
            g.phased_words = 2;
            return hip_status(launch_fused_reduce_scatter_phased(dtype, op, t, g,
                                                                 fused_lds_bytes(AR_COLL_REDUCE_SCATTER, n), stream));
        }
        return hip_status(launch_fused_reduce_scatter(dtype, op, t, g, fused_lds_bytes(AR_COLL_REDUCE_SCATTER, n),
                                                      stream));
    }
    g.W = lds_window(n);
    g.windows = (g.Rv + g.W - 1) / g.W;
    return hip_status(launch_ring_reduce_scatter(dtype, op, t, g, grid_for(g.windows, cus, 4), ring_lds_bytes(AR_COLL_REDUCE_SCATTER, n), stream));
}

ar_status_t ar_all_gather(const void *const *sendbufs, void *const *recvbufs, size_t sendcount, ar_dtype_t dtype,
                          int n, ar_sched_t sched, hipStream_t stream) {
    ar_status_t st = common_checks(sendbufs, recvbufs, dtype, AR_SUM, n, sched);
    if (st != AR_OK) return st;
    if (sendcount == 0) return AR_OK;
    if (null_entry(sendbufs, n) || null_entry((const void *const *)recvbufs, n)) return AR_ERR_INVALID_ARG;
    const size_t e = elem_size(dtype);
    if (sendcount > (SIZE_MAX / 2) / e / (size_t)n) return AR_ERR_INVALID_ARG;
    if (misaligned(sendbufs, n, e) || misaligned((const void *const *)recvbufs, n, e)) return AR_ERR_ALIGNMENT;
    uintptr_t inplace[AR_MAX_RANKS];
    for (int r = 0; r < n; ++r)
        inplace[r] = ((uintptr_t)sendbufs[r] == (uintptr_t)recvbufs[r] + (uintptr_t)r * sendcount * e) ? 1 : 0;
    st = check_overlap(sendbufs, sendcount * e, recvbufs, (size_t)n * sendcount * e, n, inplace);
    if (st != AR_OK) return st;
    ar_sched_t use;
    st = choose(AR_COLL_ALL_GATHER, sendcount, dtype, AR_SUM, n, sched, &use, (size_t)n * sendcount * e);
    if (st != AR_OK) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != AR_OK) return st;

    RankTable t;
    fill_table(t, sendbufs, recvbufs, n);
    Geometry g;
    memset(&g, 0, sizeof g);
    g.n = n;
    g.s = 1.0f;
    const bool vec = all16(sendbufs, (const void *const *)recvbufs, n) && (sendcount * e) % 16 == 0;
    if (!vec) {
        // Pieces that are not whole 16-byte vectors, or buffers off 16-byte alignment.  With every input at
        // one 16-byte phase and every output at one phase, the phased pass writes every vector of the output
        // frame (from the outputs' first 16-byte boundary) that lies wholly inside one piece, the
        // element-wise kernel the few elements at each piece's ends.  Mixed phases go element-wise.
        const long long R = (long long)sendcount, Rb = R * (long long)e;
        const int ps = one_phase(sendbufs, n), pr = one_phase((const void *const *)recvbufs, n);
        if (ps < 0 || pr < 0) {
            // Mixed phases with every pointer and the piece length whole 4-byte words: frame vector o of
            // every output is at byte 16*o and its input bytes start at a 4-byte-aligned address, all that
            // a 16-byte access needs, so the phased pass runs on the callers' pointers with one load per
            // vector and no shift; the element-wise kernel takes each piece's ends.
            if (misaligned(sendbufs, n, 4) || misaligned((const void *const *)recvbufs, n, 4) || Rb % 4 ||
                !dword_vectors())
                return hip_status(launch_elem_all_gather((int)e, t, g, R, stream));
            g.slice_bytes = Rb;
            g.phased_words = 2;
            g.ref = (long long)((uintptr_t)recvbufs[0] >> 4);
            if (aligned_tiles(Rb / 16, kFusedTile) > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;
            const hipError_t h = launch_fused_all_gather_phased(t, g, gather_lds_bytes(n, (double)n * Rb), stream);
            if (h != hipSuccess) return hip_status(h);
            return hip_status(launch_elem_all_gather_edges((int)e, t, g, R, stream));
        }
        g.slice_bytes = Rb;
        g.out_off = pr > 0 ? 16 - pr : 0;
        g.in_off = ps;
        g.last_off = ((ps + Rb - 1) >> 4) << 4;
        RankTable tp = t;
        for (int r = 0; r < n; ++r) {
            tp.src[r] = (const char *)sendbufs[r] - ps;
            tp.dst[r] = (char *)recvbufs[r] + g.out_off;
        }
        g.ref = (long long)((uintptr_t)tp.dst[0] >> 4);       // tiles follow the outputs' alignment
        if (aligned_tiles(Rb / 16, kFusedTile) > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;
        const hipError_t h = launch_fused_all_gather_phased(tp, g, gather_lds_bytes(n, (double)n * Rb), stream);
        if (h != hipSuccess) return hip_status(h);
        return hip_status(launch_elem_all_gather_edges((int)e, t, g, R, stream));
    }
    g.Rv = (long long)(sendcount * e / 16);
    g.ref = (long long)((uintptr_t)recvbufs[0] >> 4);          // fused tiles follow the outputs' alignment
    if (use == AR_SCHED_FUSED) {
        g.windows = aligned_tiles(g.Rv, kFusedTile);
        if (g.windows > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;   // grid x limit
        return hip_status(launch_fused_all_gather(t, g, gather_lds_bytes(n, (double)n * sendcount * e), stream));
    }
    g.W = lds_window(n);
    g.windows = (g.Rv + g.W - 1) / g.W;
    return hip_status(launch_ring_all_gather(t, g, grid_for(g.windows, cus, 4), ring_lds_bytes(AR_COLL_ALL_GATHER, n), stream));
}

}  // extern "C"
