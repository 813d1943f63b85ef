// tree_hi.hip -- the tree schedule's compile-time kernels for n = 9..16 (the
// kernels themselves are in tree_fast.hpp; n <= 8 is instantiated in
// tree.hip), a translation unit of its own so the two halves compile in
// parallel.
#include "tree_fast.hpp"

namespace ar {

hipError_t launch_tree_fast_hi(bool dual, int dt, int op, const RankTable &t, const TreeShape &tree,
                               const TreeShape &tree2, const Geometry &g, int lds, hipStream_t s) {
    if (dual) return launch_tree_fast_range<9, 16, true>(dt, op, t, tree, tree2, g, lds, s);
    return launch_tree_fast_range<9, 16, false>(dt, op, t, tree, tree2, g, lds, s);
}

}  // namespace ar
