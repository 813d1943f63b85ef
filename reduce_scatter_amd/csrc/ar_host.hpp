// ar_host.hpp -- host-side helpers shared by the C ABI and the planner.
#pragma once

#include <stddef.h>

#include "../../include/ar.h"
#include "ar_kernels.hpp"

namespace ar {

int tree_parent(int n, int v);
int dtree_parent(int n, int which, int v);
void tree_build(int n, TreeShape &t, int which = 0);
size_t elem_size(int dtype);
ar_status_t make_plan(ar_coll_t coll, size_t count, ar_dtype_t dtype, ar_op_t op, int n, ar_plan_t *out);
const char *calib_source();

}  // namespace ar
