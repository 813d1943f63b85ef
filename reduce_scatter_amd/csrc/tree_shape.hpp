// tree_shape.hpp -- the binary trees of the tree and double-tree schedules as
// constexpr functions of the rank count, so the host planner builds the shape
// it passes to the LDS-staged kernels and the register-evaluated kernels fold
// the same shape into their code at compile time.
//
// "NCCL all-reduce" post (rakshithvasudev.github.io), section "The double
// binary tree": in the first tree a rank's lowest set bit fixes its depth, its
// parent clears that bit and sets the next one up; the second tree swaps the
// roles of leaves and interior ranks: the mirror image of the first for even n
// (rank v takes rank n-1-v's place), the first shifted by one rank for odd n.
#pragma once

namespace ar {

constexpr int kTopoRanks = 128;

// Parent of rank v in the bit-trick tree over n ranks (rank 0 is the root).
constexpr int topo_tree_parent(int n, int v) {
    if (v <= 0 || v >= n) return -1;
    const int low = v & -v;                         // lowest set bit: fixes the depth
    int p = (v ^ low) | (low << 1);                 // clear it, set the next bit up
    if (p >= n) p = v ^ low;                        // at the edge of the range: just clear it
    return p;
}

// Parent of rank v in tree ``which`` (0: the first tree, 1: its complement).
constexpr int topo_dtree_parent(int n, int which, int v) {
    if (v < 0 || v >= n) return -1;
    if (which == 0) return topo_tree_parent(n, v);
    if (n % 2 == 0) {
        const int p = topo_tree_parent(n, n - 1 - v);
        return p < 0 ? -1 : n - 1 - p;
    }
    const int p = topo_tree_parent(n, (v + n - 1) % n);
    return p < 0 ? -1 : (p + 1) % n;
}

// The whole shape: depth, parent and up to two children per rank (-1 = none,
// in ascending rank order), the root, and post[] listing the ranks deepest
// level first (every rank after its children).
struct TreeTopo {
    int n = 0, root = 0, max_depth = 0;
    int depth[kTopoRanks] = {};
    int parent[kTopoRanks] = {};
    int child[kTopoRanks][2] = {};
    int post[kTopoRanks] = {};
};

constexpr TreeTopo tree_topo(int n, int which) {
    TreeTopo t;
    t.n = n;
    for (int v = 0; v < kTopoRanks; ++v) {
        t.parent[v] = -1;
        t.child[v][0] = t.child[v][1] = -1;
    }
    for (int v = 0; v < n; ++v) {
        int d = 0;
        for (int p = topo_dtree_parent(n, which, v); p >= 0; p = topo_dtree_parent(n, which, p)) ++d;
        t.depth[v] = d;
        if (d > t.max_depth) t.max_depth = d;
        t.parent[v] = topo_dtree_parent(n, which, v);
        if (t.parent[v] < 0) t.root = v;
    }
    for (int v = 0; v < n; ++v) {
        const int p = t.parent[v];
        if (p < 0) continue;
        if (t.child[p][0] < 0) t.child[p][0] = v;
        else t.child[p][1] = v;
    }
    int k = 0;
    for (int d = t.max_depth; d >= 0; --d)
        for (int v = 0; v < n; ++v)
            if (t.depth[v] == d) t.post[k++] = v;
    return t;
}

}  // namespace ar
