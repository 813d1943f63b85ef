// reshard_kernels.hpp -- kernel argument block of the M-to-N reshard copy
// kernel (host and device side).
//
// A reshard moves boxes of a global tensor between row-major local shards
// ("NCCL M2N" paper, arxiv.org/html/2610.07516, §IV and §V-A).  The host
// flattens every box into a segment: rows of ``row`` contiguous bytes, n0 x n1
// of them, addressed by two byte strides on each side, read once from one
// source buffer and written to ``dst_count`` destination buffers (the
// replicas of one destination shard, or one of them).  One launch carries up
// to kReshardSegs segments and a table of up to kReshardDst destination
// pointers, by value in the kernel arguments (about 3.3 KB): no device-side
// table, no allocation.
#pragma once

#include <hip/hip_runtime.h>

namespace ar {

constexpr int kReshardSegs = 24;
constexpr int kReshardDst = 128;
constexpr int kReshardThreads = 64;          // one wavefront per workgroup

struct ReshardSeg {
    const char *src;          // source buffer
    long long src_off;        // byte offset of the box's first element in the source
    long long dst_off;        // byte offset of the box's first element in every destination
    long long row;            // bytes per contiguous row (a multiple of the vector width)
    long long n1;             // rows per step of the outer dimension
    long long src_s1, dst_s1; // byte strides between consecutive rows of the middle dimension
    long long src_s0, dst_s0; // byte strides of the outer dimension
    long long tiles;          // tiles per row (kReshardThreads * u vectors each)
    long long unit0;          // first work unit of this segment within the launch
    int dst_first;            // destinations: dst[dst_first, dst_first + dst_count)
    int dst_count;
};

struct ReshardArgs {
    void *dst[kReshardDst];
    ReshardSeg seg[kReshardSegs];
    int nseg;
};

// Launch the copy of ``a`` (work units [0, units): one tile of one row each)
// with ``vb``-byte vectors (16, 8, 4, 2 or 1: every address, offset, stride
// and row length of the launch is a multiple of vb), ``u`` vectors per lane
// (1, 2, 4 or 8: tiles of 64 * u * vb bytes); ``lds`` bytes of dynamic LDS
// reserved per workgroup cap the resident workgroups per CU.
hipError_t launch_reshard(const ReshardArgs &a, long long units, int vb, int u, int lds, hipStream_t s);

}  // namespace ar
