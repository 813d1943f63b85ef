// reshard_api.cpp -- the M-to-N layout reshard: layout geometry, the
// layout-derived schedule, the leader assignment, the three routes and the
// C ABI (ar_reshard_plan, ar_reshard).
//
// Source: "NCCL M2N: A Layout- and Topology-Aware Collective for Distributed
// Tensor Resharding" (arxiv.org/html/2610.07516): §IV (layouts, Eq. (1) mesh
// ranks, Eq. (2) shard bounds, the reshard's contract), §V-A (overlap
// schedule, replicated sources collapse to one owner), §V-B (leader loads
// floor(q/rho) and one more for the first q mod rho), §V-C (the routes'
// byte volumes).  Everything is validated on the host before any launch.
#include <stdint.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/ar_reshard.h"
#include "reshard_kernels.hpp"

using namespace ar;

namespace {

constexpr int kD = AR_RESHARD_MAX_DIMS;

// Cost-model constants of the reshard routes, measured on MI355X: the copy
// kernel sustains 6.3-6.5 TB/s of HBM traffic with one read and 1-8 writes per
// byte (the MoE layer workload, every route), and a launch costs about 13 us
// from the host.
constexpr double kReshardLaunchUs = 13.0;
constexpr double kReshardGBps = 6300.0;
// Copy kernel shape, measured on MI355X at the MoE layer workload (7 GB,
// 2-8 replicas): with one vector per lane the kernel is latency-bound (2.0 TB/s
// flat, 2.8-5.2 fused); 4 vectors per lane with 8 KB of LDS reserved (at
// most 20 resident workgroups per CU) gave 6.2-6.6 TB/s for every route and
// replica count in repeated runs.  (The first process on a freshly started
// GPU runs this copy up to 20 % slower; later ones do not.)
constexpr int kReshardLdsKB = 8;
constexpr int kReshardU = 4;

struct Box {
    long long lo[kD], hi[kD];
};

bool same_box(const Box &a, const Box &b, int nd) {
    for (int d = 0; d < nd; ++d)
        if (a.lo[d] != b.lo[d] || a.hi[d] != b.hi[d]) return false;
    return true;
}

long long box_elems(const Box &b, int nd) {
    long long n = 1;
    for (int d = 0; d < nd; ++d) n *= b.hi[d] - b.lo[d];
    return n;
}

// §V-A: the per-dimension overlap [max(l), min(u)); false when any is empty.
bool overlap(const Box &a, const Box &b, int nd, Box &out) {
    for (int d = 0; d < nd; ++d) {
        out.lo[d] = std::max(a.lo[d], b.lo[d]);
        out.hi[d] = std::min(a.hi[d], b.hi[d]);
        if (out.lo[d] >= out.hi[d]) return false;
    }
    for (int d = nd; d < kD; ++d) {
        out.lo[d] = 0;
        out.hi[d] = 1;
    }
    return true;
}

int slots_of(const ar_layout_t &L) {
    int n = 1;
    for (int k = 0; k < L.mesh_ndim; ++k) n *= L.mesh[k];
    return n;
}

ar_status_t check_layout(const ar_layout_t *L) {
    if (!L) return AR_ERR_INVALID_ARG;
    if (L->ndim < 1 || L->ndim > kD || L->mesh_ndim < 1 || L->mesh_ndim > AR_RESHARD_MAX_MESH_DIMS)
        return AR_ERR_INVALID_ARG;
    for (int d = 0; d < L->ndim; ++d)
        if (L->shape[d] < 0) return AR_ERR_INVALID_ARG;
    long long slots = 1;
    for (int k = 0; k < L->mesh_ndim; ++k) {
        if (L->mesh[k] < 1 || L->mesh[k] > AR_RESHARD_MAX_SLOTS) return AR_ERR_INVALID_ARG;
        slots *= L->mesh[k];
    }
    if (slots > AR_RESHARD_MAX_SLOTS) return AR_ERR_INVALID_ARG;
    for (int k = 0; k < L->mesh_ndim; ++k) {
        const int p = L->placement[k];
        if (p != AR_REPLICATE && (p < 0 || p >= L->ndim)) return AR_ERR_INVALID_ARG;
        for (int k2 = 0; k2 < k; ++k2)
            if (p != AR_REPLICATE && L->placement[k2] == p) return AR_ERR_UNSUPPORTED;   // one axis per dimension
    }
    return AR_OK;
}

// Eq. (1): mesh coordinates of a slot (row-major) and its communicator rank.
void coords_of(const ar_layout_t &L, int slot, int *c) {
    for (int k = L.mesh_ndim - 1; k >= 0; --k) {
        c[k] = slot % L.mesh[k];
        slot /= L.mesh[k];
    }
}
int comm_rank(const ar_layout_t &L, int slot) { return L.base_rank + slot; }

// Eq. (2): the local shard of a slot.
Box shard_of(const ar_layout_t &L, int slot) {
    int c[AR_RESHARD_MAX_MESH_DIMS];
    coords_of(L, slot, c);
    Box b;
    for (int d = 0; d < kD; ++d) {
        b.lo[d] = 0;
        b.hi[d] = d < L.ndim ? L.shape[d] : 1;
    }
    for (int k = 0; k < L.mesh_ndim; ++k) {
        const int d = L.placement[k];
        if (d == AR_REPLICATE) continue;
        const long long S = L.shape[d], D = L.mesh[k];
        b.lo[d] = (long long)c[k] * S / D;          // c < 128 and S <= 2^40: no overflow
        b.hi[d] = (long long)(c[k] + 1) * S / D;
    }
    return b;
}

// Everything derived from the two layouts: shards, owners, destination
// shards with their replica slots, contributions per shard.
struct ReshardGeo {
    int nd = 0;
    int nsrc = 0, ndst = 0;
    std::vector<Box> src_box, dst_box;
    std::vector<int> owners;                 // owner source slots, ascending
    std::vector<std::vector<int>> replicas;  // per destination shard j: its slots, ascending
    std::vector<int> shard_of_slot;          // destination slot -> j
    std::vector<std::vector<int>> contrib;   // per j: owner slots overlapping it, ascending
    long long unique_elems = 0;
};

ar_status_t derive(const ar_layout_t *src, const ar_layout_t *dst, size_t elem_size, ReshardGeo &g) {
    ar_status_t st = check_layout(src);
    if (st != AR_OK) return st;
    st = check_layout(dst);
    if (st != AR_OK) return st;
    if (src->ndim != dst->ndim) return AR_ERR_INVALID_ARG;
    long long total = 1;
    for (int d = 0; d < src->ndim; ++d) {
        if (src->shape[d] != dst->shape[d]) return AR_ERR_INVALID_ARG;   // one global shape
        if (src->shape[d] > (1LL << 40)) return AR_ERR_INVALID_ARG;
        total = total > 0 && src->shape[d] > 0 ? total * src->shape[d] : 0;
        if (total > (1LL << 50)) return AR_ERR_INVALID_ARG;
    }
    if (elem_size != 1 && elem_size != 2 && elem_size != 4 && elem_size != 8 && elem_size != 16)
        return AR_ERR_UNSUPPORTED;
    g.nd = src->ndim;
    g.nsrc = slots_of(*src);
    g.ndst = slots_of(*dst);
    for (int s = 0; s < g.nsrc; ++s) g.src_box.push_back(shard_of(*src, s));
    for (int t = 0; t < g.ndst; ++t) g.dst_box.push_back(shard_of(*dst, t));
    for (int s = 0; s < g.nsrc; ++s) {                    // the lowest slot of every set of replicas
        bool first = true;
        for (int s2 = 0; s2 < s && first; ++s2)
            if (same_box(g.src_box[s2], g.src_box[s], g.nd)) first = false;
        if (first) g.owners.push_back(s);
    }
    g.shard_of_slot.assign(g.ndst, -1);
    for (int t = 0; t < g.ndst; ++t) {
        for (size_t j = 0; j < g.replicas.size(); ++j)
            if (same_box(g.dst_box[g.replicas[j][0]], g.dst_box[t], g.nd)) {
                g.shard_of_slot[t] = (int)j;
                break;
            }
        if (g.shard_of_slot[t] < 0) {
            g.shard_of_slot[t] = (int)g.replicas.size();
            g.replicas.push_back({});
        }
        g.replicas[g.shard_of_slot[t]].push_back(t);
    }
    g.contrib.resize(g.replicas.size());
    for (size_t j = 0; j < g.replicas.size(); ++j) {
        const Box &bj = g.dst_box[g.replicas[j][0]];
        g.unique_elems += box_elems(bj, g.nd);
        Box o;
        for (int s : g.owners)
            if (overlap(g.src_box[s], bj, g.nd, o)) g.contrib[j].push_back(s);
    }
    return AR_OK;
}

// §V-B: the leader (destination slot) of contribution i (index into
// contrib[j]) of shard j, with the replicas split evenly over ``domains``.
int leader_slot(const ReshardGeo &g, int j, int i, int domains) {
    const int rho = (int)g.replicas[j].size() / domains;
    const int q = (int)g.contrib[j].size();
    const int a = q / rho, b = q % rho;
    // replica r takes contributions [r*a + min(r, b), (r+1)*a + min(r+1, b))
    for (int r = 0; r < rho; ++r) {
        const int end = (r + 1) * a + std::min(r + 1, b);
        if (i < end) return g.replicas[j][r];
    }
    return g.replicas[j][rho - 1];
}

// A box as a segment: rows of contiguous bytes in both buffers.  ``sb`` and
// ``db`` are the shards (local extents and origins) of the source and
// destination buffers.
struct Flat {
    long long src_off, dst_off, row, n0, n1, src_s0, src_s1, dst_s0, dst_s1;
};

Flat flatten(const Box &box, const Box &sb, const Box &db, int nd, long long e) {
    long long es[kD], et[kD], ss[kD], st[kD], ext[kD];
    for (int d = 0; d < nd; ++d) {
        es[d] = sb.hi[d] - sb.lo[d];
        et[d] = db.hi[d] - db.lo[d];
        ext[d] = box.hi[d] - box.lo[d];
    }
    ss[nd - 1] = st[nd - 1] = 1;
    for (int d = nd - 2; d >= 0; --d) {
        ss[d] = ss[d + 1] * es[d + 1];
        st[d] = st[d + 1] * et[d + 1];
    }
    Flat f;
    f.src_off = f.dst_off = 0;
    for (int d = 0; d < nd; ++d) {
        f.src_off += (box.lo[d] - sb.lo[d]) * ss[d];
        f.dst_off += (box.lo[d] - db.lo[d]) * st[d];
    }
    // merge trailing dimensions while the box spans them whole on both sides
    long long run = ext[nd - 1];
    int d = nd - 2;
    while (d >= 0 && ext[d + 1] == es[d + 1] && ext[d + 1] == et[d + 1]) {
        run *= ext[d];
        --d;
    }
    // dimensions 0..d remain as row loops (at most two)
    f.n0 = f.n1 = 1;
    f.src_s0 = f.src_s1 = f.dst_s0 = f.dst_s1 = 0;
    if (d == 0) {
        f.n1 = ext[0];
        f.src_s1 = ss[0] * e;
        f.dst_s1 = st[0] * e;
    } else if (d == 1) {
        f.n0 = ext[0];
        f.src_s0 = ss[0] * e;
        f.dst_s0 = st[0] * e;
        f.n1 = ext[1];
        f.src_s1 = ss[1] * e;
        f.dst_s1 = st[1] * e;
    }
    f.row = run * e;
    f.src_off *= e;
    f.dst_off *= e;
    return f;
}

// One segment of a route before it is packed into launches.
struct Piece {
    Flat f;
    const char *src;
    int shard;                 // the destination table of its launch: the replicas of this shard
    int dst_first, dst_count;  // within that table
};

// Pack pieces (all of one shard's table, in order) into launches.
ar_status_t run_pieces(const std::vector<Piece> &pieces, const std::vector<void *> &table, int vb, int u, int lds,
                       hipStream_t stream, int *launches) {
    ReshardArgs a;
    memset(&a, 0, sizeof a);
    for (size_t i = 0; i < table.size(); ++i) a.dst[i] = table[i];
    long long units = 0;
    auto flush = [&]() -> ar_status_t {
        if (a.nseg == 0) return AR_OK;
        hipError_t e = launch_reshard(a, units, vb, u, lds, stream);
        if (launches) ++*launches;
        a.nseg = 0;
        units = 0;
        return e == hipSuccess ? AR_OK : AR_ERR_HIP;
    };
    const long long tile_bytes = (long long)kReshardThreads * u * vb;
    for (const Piece &p : pieces) {
        if (p.dst_count == 0) continue;
        const long long tiles = (p.f.row + tile_bytes - 1) / tile_bytes;
        const long long n = tiles * p.f.n0 * p.f.n1;
        if (n <= 0) continue;
        if (n > 0x7fffffffLL) return AR_ERR_UNSUPPORTED;       // one box of more than 2^31 tiles
        if (a.nseg == kReshardSegs || units + n > 0x7fffffffLL) {
            ar_status_t st = flush();
            if (st != AR_OK) return st;
        }
        ReshardSeg &s = a.seg[a.nseg++];
        s.src = p.src;
        s.src_off = p.f.src_off;
        s.dst_off = p.f.dst_off;
        s.row = p.f.row;
        s.n1 = p.f.n1;
        s.src_s1 = p.f.src_s1;
        s.dst_s1 = p.f.dst_s1;
        s.src_s0 = p.f.src_s0;
        s.dst_s0 = p.f.dst_s0;
        s.tiles = tiles;
        s.unit0 = units;
        s.dst_first = p.dst_first;
        s.dst_count = p.dst_count;
        units += n;
    }
    return flush();
}

// The pieces of a route, per destination shard, in two phases (the second
// runs after the first: the hierarchical route's fan-out from the leaders).
// With null buffer arrays only the counts are meaningful.
struct Pieces {
    std::vector<std::vector<Piece>> phase[2];
};

void build_pieces(const ReshardGeo &g, ar_route_t use, const void *const *src_bufs, void *const *dst_bufs,
                  long long e, Pieces &out) {
    for (auto &ph : out.phase) ph.assign(g.replicas.size(), {});
    for (size_t j = 0; j < g.replicas.size(); ++j) {
        const std::vector<int> &rep = g.replicas[j];
        const Box &bj = g.dst_box[rep[0]];
        for (size_t i = 0; i < g.contrib[j].size(); ++i) {
            const int s = g.contrib[j][i];
            Box o;
            overlap(g.src_box[s], bj, g.nd, o);
            Piece p;
            p.f = flatten(o, g.src_box[s], bj, g.nd, e);
            p.src = src_bufs ? (const char *)src_bufs[s] : nullptr;
            p.shard = (int)j;
            if (use == AR_ROUTE_FUSED) {                        // one read, every replica written
                p.dst_first = 0;
                p.dst_count = (int)rep.size();
                out.phase[0][j].push_back(p);
            } else if (use == AR_ROUTE_FLAT) {                  // one read per replica
                for (size_t r = 0; r < rep.size(); ++r) {
                    p.dst_first = (int)r;
                    p.dst_count = 1;
                    out.phase[0][j].push_back(p);
                }
            } else {                                            // hierarchical: leader, then fan-out
                const int lead = leader_slot(g, (int)j, (int)i, 1);
                const int li = (int)(std::find(rep.begin(), rep.end(), lead) - rep.begin());
                p.dst_first = li;
                p.dst_count = 1;
                out.phase[0][j].push_back(p);
                Piece q = p;
                q.f = flatten(o, bj, bj, g.nd, e);
                q.src = dst_bufs ? (const char *)dst_bufs[lead] : nullptr;
                if (li > 0) {                                   // replicas before the leader
                    q.dst_first = 0;
                    q.dst_count = li;
                    out.phase[1][j].push_back(q);
                }
                if (li + 1 < (int)rep.size()) {                 // and after it
                    q.dst_first = li + 1;
                    q.dst_count = (int)rep.size() - li - 1;
                    out.phase[1][j].push_back(q);
                }
            }
        }
    }
}

// Route volumes (§V-C with every replica in one domain) and launch counts
// (pieces packed kReshardSegs to a launch, one destination table each).
void route_costs(const ReshardGeo &g, size_t e, ar_reshard_plan_t *out) {
    double vol[4] = {0, 0, 0, 0};
    for (size_t j = 0; j < g.replicas.size(); ++j) {
        const double bj = (double)box_elems(g.dst_box[g.replicas[j][0]], g.nd) * (double)e;
        const double r = (double)g.replicas[j].size();
        vol[AR_ROUTE_FLAT] += 2.0 * r * bj;
        vol[AR_ROUTE_HIER] += (2.0 + r) * bj;
        vol[AR_ROUTE_FUSED] += (1.0 + r) * bj;
    }
    int best = AR_ROUTE_FUSED;
    for (int r = AR_ROUTE_FLAT; r <= AR_ROUTE_FUSED; ++r) {
        Pieces pc;
        build_pieces(g, (ar_route_t)r, nullptr, nullptr, (long long)e, pc);
        int launches = 0;
        for (auto &ph : pc.phase)
            for (auto &v : ph) launches += (int)((v.size() + kReshardSegs - 1) / kReshardSegs);
        out->bytes[r] = vol[r];
        out->launches[r] = launches;
        out->predicted_us[r] = launches * kReshardLaunchUs + vol[r] / (kReshardGBps * 1e3);
        if (out->predicted_us[r] < out->predicted_us[best]) best = r;
    }
    out->chosen = (ar_route_t)best;
}

int reshard_lds_bytes() {
    static const int v = [] {
        const char *e = getenv("AR_RESHARD_LDS_KB");
        const long kb = (e && *e) ? atol(e) : kReshardLdsKB;
        return (int)std::min(std::max(kb, 0L), 64L) * 1024;
    }();
    return v;
}

// Vectors per lane of the copy kernel (AR_RESHARD_U overrides: 1, 2, 4, 8).
int reshard_u() {
    static const int v = [] {
        const char *e = getenv("AR_RESHARD_U");
        const long x = (e && *e) ? atol(e) : kReshardU;
        return (x == 1 || x == 2 || x == 4 || x == 8) ? (int)x : kReshardU;
    }();
    return v;
}

}  // namespace

extern "C" {

ar_status_t ar_layout_shard(const ar_layout_t *layout, int slot, long long *lo, long long *hi, int *rank) {
    ar_status_t st = check_layout(layout);
    if (st != AR_OK) return st;
    if (!lo || !hi || slot < 0 || slot >= slots_of(*layout)) return AR_ERR_INVALID_ARG;
    const Box b = shard_of(*layout, slot);
    for (int d = 0; d < kD; ++d) {
        lo[d] = b.lo[d];
        hi[d] = b.hi[d];
    }
    if (rank) *rank = comm_rank(*layout, slot);
    return AR_OK;
}

ar_status_t ar_reshard_plan(const ar_layout_t *src, const ar_layout_t *dst, size_t elem_size, int domains,
                            ar_reshard_plan_t *out, ar_transfer_t *transfers, int max_transfers) {
    if (!out || domains < 1 || max_transfers < 0) return AR_ERR_INVALID_ARG;
    ReshardGeo g;
    ar_status_t st = derive(src, dst, elem_size, g);
    if (st != AR_OK) return st;
    for (auto &r : g.replicas)
        if ((int)r.size() % domains) return AR_ERR_INVALID_ARG;
    memset(out, 0, sizeof *out);
    out->n_sources = (int)g.owners.size();
    out->n_shards = (int)g.replicas.size();
    for (auto &r : g.replicas) out->max_replicas = std::max(out->max_replicas, (int)r.size());
    out->unique_bytes = g.unique_elems * (long long)elem_size;
    route_costs(g, elem_size, out);
    int n = 0;
    for (int s : g.owners) {
        for (int t = 0; t < g.ndst; ++t) {
            Box o;
            if (!overlap(g.src_box[s], g.dst_box[t], g.nd, o)) continue;
            if (transfers && n < max_transfers) {
                ar_transfer_t &x = transfers[n];
                const int j = g.shard_of_slot[t];
                const int i = (int)(std::find(g.contrib[j].begin(), g.contrib[j].end(), s) - g.contrib[j].begin());
                x.src_rank = comm_rank(*src, s);
                x.dst_rank = comm_rank(*dst, t);
                x.leader_rank = comm_rank(*dst, leader_slot(g, j, i, domains));
                for (int d = 0; d < kD; ++d) {
                    x.lo[d] = o.lo[d];
                    x.hi[d] = o.hi[d];
                }
                x.bytes = box_elems(o, g.nd) * (long long)elem_size;
            }
            ++n;
        }
    }
    out->n_transfers = n;
    return AR_OK;
}

ar_status_t ar_reshard(const void *const *src_bufs, void *const *dst_bufs, const ar_layout_t *src,
                       const ar_layout_t *dst, size_t elem_size, ar_route_t route, hipStream_t stream) {
    if (!src_bufs || !dst_bufs) return AR_ERR_INVALID_ARG;
    if (route < AR_ROUTE_AUTO || route > AR_ROUTE_FUSED) return AR_ERR_INVALID_ARG;
    ReshardGeo g;
    ar_status_t st = derive(src, dst, elem_size, g);
    if (st != AR_OK) return st;
    const long long e = (long long)elem_size;
    // buffers: owners and destinations non-null (unless their shard is empty) and element-aligned
    for (int s : g.owners) {
        if (!src_bufs[s] && box_elems(g.src_box[s], g.nd) > 0) return AR_ERR_INVALID_ARG;
        if ((uintptr_t)src_bufs[s] % elem_size) return AR_ERR_ALIGNMENT;
    }
    for (int t = 0; t < g.ndst; ++t) {
        if (!dst_bufs[t] && box_elems(g.dst_box[t], g.nd) > 0) return AR_ERR_INVALID_ARG;
        if ((uintptr_t)dst_bufs[t] % elem_size) return AR_ERR_ALIGNMENT;
    }
    // no destination range may overlap another destination or a source that is read
    struct Range {
        uintptr_t lo, hi;
        bool dst;
    };
    std::vector<Range> rs;
    for (int s : g.owners) {
        const uintptr_t n = (uintptr_t)(box_elems(g.src_box[s], g.nd) * e);
        if (n) rs.push_back({(uintptr_t)src_bufs[s], (uintptr_t)src_bufs[s] + n, false});
    }
    for (int t = 0; t < g.ndst; ++t) {
        const uintptr_t n = (uintptr_t)(box_elems(g.dst_box[t], g.nd) * e);
        if (n) rs.push_back({(uintptr_t)dst_bufs[t], (uintptr_t)dst_bufs[t] + n, true});
    }
    std::sort(rs.begin(), rs.end(), [](const Range &a, const Range &b) { return a.lo < b.lo; });
    uintptr_t end_any = 0, end_dst = 0;
    for (const Range &r : rs) {
        if (r.lo < (r.dst ? end_any : end_dst)) return AR_ERR_INVALID_ARG;
        end_any = std::max(end_any, r.hi);
        if (r.dst) end_dst = std::max(end_dst, r.hi);
    }
    if (g.unique_elems == 0) return AR_OK;

    ar_reshard_plan_t costs;
    memset(&costs, 0, sizeof costs);
    route_costs(g, elem_size, &costs);
    const ar_route_t use = route == AR_ROUTE_AUTO ? costs.chosen : route;

    Pieces pc;
    build_pieces(g, use, src_bufs, dst_bufs, e, pc);
    // vector width: the largest power of two <= 16 dividing every address,
    // offset, stride and row length the launches use
    uintptr_t bits = 16;
    auto fold = [&](uintptr_t v) { bits |= v; };
    for (size_t j = 0; j < g.replicas.size(); ++j) {
        for (int t : g.replicas[j]) fold((uintptr_t)dst_bufs[t]);
        for (auto &ph : pc.phase)
            for (const Piece &p : ph[j]) {
                fold((uintptr_t)p.src);
                fold((uintptr_t)p.f.src_off);
                fold((uintptr_t)p.f.dst_off);
                fold((uintptr_t)p.f.row);
                fold((uintptr_t)p.f.src_s0);
                fold((uintptr_t)p.f.src_s1);
                fold((uintptr_t)p.f.dst_s0);
                fold((uintptr_t)p.f.dst_s1);
            }
    }
    const int vb = (int)(bits & (~bits + 1));                    // lowest set bit, at most 16
    const int lds = reshard_lds_bytes();
    for (auto &ph : pc.phase) {
        for (size_t j = 0; j < g.replicas.size(); ++j) {
            std::vector<void *> table;
            for (int t : g.replicas[j]) table.push_back(dst_bufs[t]);
            st = run_pieces(ph[j], table, vb, reshard_u(), lds, stream, nullptr);
            if (st != AR_OK) return st;
        }
    }
    return AR_OK;
}

}  // extern "C"
