// plan.cpp -- the cost model that picks a schedule per call, and the tree
// builder.  Host code only (no HIP calls), so it runs without a GPU.
//
// Cost model: the "NCCL all-reduce" post (rakshithvasudev.github.io), section
// "How NCCL picks: a cost model, not a threshold": every legal algorithm is
// priced as latency plus bytes over bandwidth and the cheapest one wins, per
// call; there is no size threshold.  Tables of measured constants are filled
// once at start-up; a candidate the hardware cannot run is simply absent
// (section "What your hardware takes off the menu").  Here:
//
//   t_s = launch_us[s] + step_us[s] * steps_s(n) + bytes_s / bandwidth_s(bytes)
//
//   steps:  ring 2(n-1) for all-reduce, n-1 for reduce-scatter / all-gather
//           (section "The ring, exactly as the kernel runs it"); tree
//           2 * depth (section "The double binary tree"), the same for the
//           double tree; fused 1; split 1 (one pass; its log-depth combine
//           stays inside a workgroup).
//   bytes:  the algorithmic HBM bytes.  All three schedules keep partial
//           results on chip, so each moves 2*n*S for an all-reduce of S bytes
//           per rank, (n+1)*n*R*e for reduce-scatter and all-gather.
//   bandwidth_s(bytes): a measured sustained rate times a measured per-size
//           correction (the role of the tree correction table in the same
//           section: the clean model does not fit medium sizes, so a
//           per-size factor is applied), indexed by the call's total bytes.
//
// Legality: the tree, double-tree and split schedules exist for all-reduce only.
//
// Constants come from a calibration file (AR_CALIB, default
// calib_gfx950.txt beside the library) written by the package's calibration
// script from timed runs; built-in defaults apply when it is missing.
#include <dlfcn.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/ar.h"
#include "ar_host.hpp"
#include "tree_shape.hpp"

static_assert(ar::kTopoRanks == ar::kTableRanks, "tree shapes cover the rank table");

// Predicted-time margin within which the fused schedule is kept, for calls
// whose footprint is at least kHbmBytes (see make_plan).
constexpr double kTieMargin = 0.03;
constexpr double kHbmBytes = 1073741824.0;
constexpr double kTieUs = 0.5;              // ... and within this many microseconds at any footprint

namespace ar {

namespace {

constexpr int kColls = 3;
constexpr int kScheds = 6;         // indexed by ar_sched_t; 0 (auto) unused
constexpr int kSizeBins = 48;      // per-size correction for log2(algorithmic bytes of the call) = 0..47

// Rank classes: ceil(log2 n) = 0..7 for n = 1..96, and 8 for 97..128.  The
// top octave is split because the schedules rank differently across it: at
// 72 ranks split led the one-pass schedules on most boxes, at 128 (8 MB per
// rank) fused led split by up to 10 %, and one class averaged the two.
constexpr int kRankClasses = 9;

// Bandwidth of one element-size class: a sustained rate and the per-(rank
// class, footprint) correction.  4-byte types (fp32, int32) and 2-byte types
// (bf16, fp16) have tables of their own: the per-element work differs (bf16 and
// fp16 partials are rounded at every hop, the ring stages twice the elements
// per byte through LDS), so schedules that tie in fp32 can differ in bf16.
struct Bandwidth {
    double bw_gbps = 0;
    double corr[kRankClasses][kSizeBins];
    bool measured[kRankClasses];       // a corr row was read for this rank class
};

struct Entry {
    double launch_us = 0, step_us = 0;
    Bandwidth b4, b2;                  // 4-byte and 2-byte element types
    bool have_b2 = false;              // a 2-byte rate was read (else 2-byte calls use b4)
    double extra_us[kRankClasses];     // measured latency beyond launch + step * steps, per rank class
    bool lat_read[kRankClasses];       // a lat row was read for this rank class
    bool set = false;
};

struct Calib {
    Entry e[kColls][kScheds];
    std::string source = "defaults";
};

Calib g_calib;
std::once_flag g_calib_once;

void set_defaults(Calib &c) {
    // Conservative start-up constants for MI355X (replaced by the measured
    // file when present): a few microseconds of launch cost, a workgroup
    // barrier per dependent step, and HBM-class streaming bandwidth.
    for (int k = 0; k < kColls; ++k)
        for (int s = 1; s < kScheds; ++s) {
            Entry &e = c.e[k][s];
            e.launch_us = 8.0;
            const bool one_pass = s == AR_SCHED_FUSED || s == AR_SCHED_SPLIT;
            e.step_us = one_pass ? 0.0 : 0.25;
            for (Bandwidth *bw : {&e.b4, &e.b2}) {
                bw->bw_gbps = s == AR_SCHED_FUSED ? 5000.0 : 4000.0;
                for (int k2 = 0; k2 < kRankClasses; ++k2) {
                    bw->measured[k2] = false;
                    for (int b = 0; b < kSizeBins; ++b) bw->corr[k2][b] = 1.0;
                }
            }
            e.have_b2 = false;
            for (int k2 = 0; k2 < kRankClasses; ++k2) {
                e.extra_us[k2] = 0.0;
                e.lat_read[k2] = false;
            }
            e.set = true;
        }
}

int coll_index(const char *s) {
    if (!strcmp(s, "allreduce")) return AR_COLL_ALLREDUCE;
    if (!strcmp(s, "reduce_scatter")) return AR_COLL_REDUCE_SCATTER;
    if (!strcmp(s, "all_gather")) return AR_COLL_ALL_GATHER;
    return -1;
}

int sched_index(const char *s) {
    if (!strcmp(s, "ring")) return AR_SCHED_RING;
    if (!strcmp(s, "tree")) return AR_SCHED_TREE;
    if (!strcmp(s, "fused")) return AR_SCHED_FUSED;
    if (!strcmp(s, "split")) return AR_SCHED_SPLIT;
    if (!strcmp(s, "dtree")) return AR_SCHED_DTREE;
    return -1;
}

std::string library_dir() {
    Dl_info info;
    if (dladdr((void *)&library_dir, &info) && info.dli_fname) {
        std::string p(info.dli_fname);
        size_t k = p.rfind('/');
        if (k != std::string::npos) return p.substr(0, k);
    }
    return ".";
}

// File format, one record per line ('#' starts a comment):
//   <coll> <sched> <launch_us> <step_us> <bw_gbps>
//   corr <coll> <sched> <rank class> <corr_0 ... corr_47>
//   lat <coll> <sched> <rank class> <extra_us>
//   bw2 <coll> <sched> <bw_gbps>                     (2-byte element types)
//   corr2 <coll> <sched> <rank class> <corr_0 ... corr_47>
// coll in {allreduce, reduce_scatter, all_gather}, sched in {ring, tree, fused, split, dtree};
// rank class = ceil(log2 n); corr_b multiplies the bandwidth for calls that
// move 2^b .. 2^(b+1)-1 algorithmic bytes in total (the footprint decides
// whether the data stays in the 256 MB Infinity Cache, and how that bends the
// bandwidth depends on n).  A rank class without a row uses the nearest one
// that has one.  extra_us is added to the latency of calls in that rank class
// (kernels for different rank counts do not share one per-step cost).
void load_file(Calib &c, const std::string &path) {
    FILE *f = fopen(path.c_str(), "r");
    if (!f) return;
    char line[2048];
    int loaded = 0;
    while (fgets(line, sizeof line, f)) {
        char *hash = strchr(line, '#');
        if (hash) *hash = 0;
        char coll[32], sched[32];
        int used = 0, rc = -1;
        double lu, su, bw;
        double extra = 0;
        if (sscanf(line, "lat %31s %31s %d %lf", coll, sched, &rc, &extra) == 4) {
            int k = coll_index(coll), s = sched_index(sched);
            if (k >= 0 && s >= 0 && rc >= 0 && rc < kRankClasses) {
                c.e[k][s].extra_us[rc] = extra;
                c.e[k][s].lat_read[rc] = true;
            }
            continue;
        }
        if (sscanf(line, "bw2 %31s %31s %lf", coll, sched, &bw) == 3) {
            int k = coll_index(coll), s = sched_index(sched);
            if (k >= 0 && s >= 0 && bw > 0) {
                c.e[k][s].b2.bw_gbps = bw;
                c.e[k][s].have_b2 = true;
            }
            continue;
        }
        const bool two = strncmp(line, "corr2 ", 6) == 0;
        if ((two && sscanf(line, "corr2 %31s %31s %d%n", coll, sched, &rc, &used) == 3) ||
            (!two && sscanf(line, "corr %31s %31s %d%n", coll, sched, &rc, &used) == 3)) {
            int k = coll_index(coll), s = sched_index(sched);
            if (k < 0 || s < 0 || rc < 0 || rc >= kRankClasses) continue;
            Bandwidth &bt = two ? c.e[k][s].b2 : c.e[k][s].b4;
            const char *p = line + used;
            for (int b = 0; b < kSizeBins; ++b) {
                double v;
                int m = 0;
                if (sscanf(p, "%lf%n", &v, &m) != 1) break;
                if (v > 0) bt.corr[rc][b] = v;
                p += m;
            }
            bt.measured[rc] = true;
            continue;
        }
        if (sscanf(line, "%31s %31s %lf %lf %lf%n", coll, sched, &lu, &su, &bw, &used) != 5) continue;
        int k = coll_index(coll), s = sched_index(sched);
        if (k < 0 || s < 0 || !(bw > 0) || lu < 0 || su < 0) continue;
        Entry &e = c.e[k][s];
        e.launch_us = lu;
        e.step_us = su;
        e.b4.bw_gbps = bw;
        ++loaded;
    }
    fclose(f);
    if (loaded) c.source = path;
}

void init_calib() {
    set_defaults(g_calib);
    const char *env = getenv("AR_CALIB");
    load_file(g_calib, env && *env ? std::string(env) : library_dir() + "/calib_gfx950.txt");
}

int rank_class(int n) {
    int k = 0;
    while ((1 << k) < n) ++k;
    if (k >= 7) return n > 96 ? 8 : 7;
    return k;
}

// The measured correction row nearest to rank class k (nullptr if none).
const double *corr_row(const Bandwidth &b, int k) {
    for (int d = 0; d < kRankClasses; ++d) {
        if (k - d >= 0 && b.measured[k - d]) return b.corr[k - d];
        if (k + d < kRankClasses && b.measured[k + d]) return b.corr[k + d];
    }
    return nullptr;
}

// Latency beyond launch + step * steps for rank class k: the class's own term
// where the calibration measured the class (a lat or corr row; zero if it
// wrote no lat row, having found none worth writing), else that of the
// nearest measured class.
double extra_latency(const Entry &e, int k) {
    const auto measured = [&](int j) { return e.lat_read[j] || e.b4.measured[j]; };
    for (int d = 0; d < kRankClasses; ++d) {
        if (k - d >= 0 && measured(k - d)) return e.extra_us[k - d];
        if (k + d < kRankClasses && measured(k + d)) return e.extra_us[k + d];
    }
    return 0.0;
}

// Bandwidth (GB/s) of schedule entry ``e`` for a call of element size ``elem``
// bytes, rank class k and footprint bin ``bin``.  2-byte calls take the 2-byte
// rate when one was measured, with the 2-byte correction (else the 4-byte one);
// everything else takes the 4-byte table.  A rank class without a row uses the
// nearest measured one (all ones when none is).
double bandwidth(const Entry &e, int elem, int k, int bin) {
    const bool two = elem == 2 && e.have_b2;
    const double *row = two ? corr_row(e.b2, k) : nullptr;
    if (!row) row = corr_row(e.b4, k);
    return (two ? e.b2.bw_gbps : e.b4.bw_gbps) * (row ? row[bin] : 1.0);
}

int size_bin(double bytes) {
    if (bytes < 1) return 0;
    int b = (int)std::floor(std::log2(bytes));
    return b < 0 ? 0 : (b >= kSizeBins ? kSizeBins - 1 : b);
}

}  // namespace

int tree_parent(int n, int v) { return topo_tree_parent(n, v); }

int dtree_parent(int n, int which, int v) { return topo_dtree_parent(n, which, v); }

void tree_build(int n, TreeShape &t, int which) {
    const TreeTopo s = tree_topo(n, which);
    memset(&t, 0, sizeof t);
    for (int v = 0; v < kTableRanks; ++v) {
        t.depth[v] = (int8_t)s.depth[v];
        t.parent[v] = (int8_t)s.parent[v];
        t.child[v][0] = (int8_t)s.child[v][0];
        t.child[v][1] = (int8_t)s.child[v][1];
        t.post[v] = (uint8_t)s.post[v];
    }
    t.max_depth = s.max_depth;
    t.root = s.root;
}

size_t elem_size(int dtype) { return (dtype == AR_BFLOAT16 || dtype == AR_FLOAT16) ? 2 : 4; }

ar_status_t make_plan(ar_coll_t coll, size_t count, ar_dtype_t dtype, ar_op_t op, int n, ar_plan_t *out) {
    (void)op;
    std::call_once(g_calib_once, init_calib);
    memset(out, 0, sizeof *out);
    const double e = (double)elem_size(dtype);
    double bytes = 0, per_rank = 0;
    if (coll == AR_COLL_ALLREDUCE) {
        per_rank = (double)count * e;
        bytes = 2.0 * n * per_rank;
    } else {                                        // RS: n*R in, R out; AG: R in, n*R out
        per_rank = (double)n * count * e;
        bytes = (n + 1.0) * n * (double)count * e;
    }
    int depth = 0;                                  // the bit-trick tree over n ranks is ceil(log2 n) deep
    while ((1 << depth) < n) ++depth;
    out->legal_mask = (1u << AR_SCHED_RING) | (1u << AR_SCHED_FUSED);
    if (coll == AR_COLL_ALLREDUCE)
        out->legal_mask |= (1u << AR_SCHED_TREE) | (1u << AR_SCHED_SPLIT) | (1u << AR_SCHED_DTREE);
    out->steps[AR_SCHED_RING] = (coll == AR_COLL_ALLREDUCE) ? 2 * (n - 1) : (n - 1);
    out->steps[AR_SCHED_TREE] = (coll == AR_COLL_ALLREDUCE) ? 2 * depth : 0;
    out->steps[AR_SCHED_FUSED] = 1;
    out->steps[AR_SCHED_SPLIT] = (coll == AR_COLL_ALLREDUCE) ? 1 : 0;
    out->steps[AR_SCHED_DTREE] = out->steps[AR_SCHED_TREE];
    double best = 0;
    out->chosen = AR_SCHED_FUSED;
    bool have = false;
    (void)per_rank;
    const int bin = size_bin(bytes);
    const int rclass = rank_class(n);
    for (int s = AR_SCHED_RING; s <= AR_SCHED_DTREE; ++s) {
        if (!(out->legal_mask & (1u << s))) continue;
        const Entry &c = g_calib.e[coll][s];
        out->bytes[s] = bytes;
        const double bw = bandwidth(c, (int)e, rclass, bin);       // GB/s = 1e3 bytes per microsecond
        out->predicted_us[s] = c.launch_us + c.step_us * out->steps[s] + extra_latency(c, rclass) + bytes / (bw * 1e3);
        if (!have || out->predicted_us[s] < best) {
            best = out->predicted_us[s];
            out->chosen = (ar_sched_t)s;
            have = true;
        }
    }
    // Calls that stream from HBM (a footprint of kHbmBytes or more, four times the 256 MB Infinity Cache):
    // schedules that move the same bytes in one pass (fused, tree and dtree in registers, split) run within a
    // few per cent of one another there, less than the spread between calibration runs and boxes, so one
    // preferred schedule keeps the call unless another is predicted faster by more than kTieMargin.  Below
    // that footprint the differences between them are real (at 16 ranks and 16 MB per rank, half in the cache,
    // the trees ran 8-12 % ahead of fused on two boxes) and the argmin stands.  At every footprint, a
    // predicted advantage under kTieUs is below the launch-to-launch jitter of about a microsecond (calls
    // under 1 MB per rank all take 8-11 us whatever the schedule), so the preferred schedule keeps the call.
    // The preferred schedule is fused, whose pass needs no cross-wave exchange, up to 16 ranks, and split past
    // 16 where it is legal: there the two differ by less than the allocation moves either (72 ranks, 25 MB per
    // rank, one box: 67-77 % of peak for split and 67-73 % for fused across fresh sets of buffers), and at the
    // bucketed workload's sizes split ran ahead on most boxes (by 1-5 %).
    const ar_sched_t pref = (n > 16 && (out->legal_mask & (1u << AR_SCHED_SPLIT))) ? AR_SCHED_SPLIT : AR_SCHED_FUSED;
    if (have && out->chosen != pref &&
        (out->predicted_us[pref] <= best + kTieUs ||
         (bytes >= kHbmBytes && out->predicted_us[pref] <= best * (1.0 + kTieMargin))))
        out->chosen = pref;
    return AR_OK;
}

const char *calib_source() {
    std::call_once(g_calib_once, init_calib);
    return g_calib.source.c_str();
}

}  // namespace ar
