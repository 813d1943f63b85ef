/*
 * ar_oracle.c -- CPU oracle for the n-rank all-reduce / reduce-scatter /
 * all-gather path.  TEST INFRASTRUCTURE ONLY: nothing in the product library
 * may include, link or call this file; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header or table
 * with the GPU path.
 *
 * Plain, slow and literal on purpose: ranks are simulated one by one, each
 * ring step moves whole chunk messages between per-rank "wire" buffers, and
 * every element goes through a per-element switch on dtype and op.  The only
 * concession to speed is an OpenMP loop over the elements of one message,
 * which leaves every element's own sequence of operations unchanged, so the
 * results are identical at any thread count.
 *
 * Sources (the pages these functions follow):
 *  [AR]  "NCCL all-reduce" post, rakshithvasudev.github.io (feed):
 *        sections "What all-reduce promises" (contract, ops, avg rule),
 *        "The ring, exactly as the kernel runs it" (n chunks, n-1 reduce
 *        hops, n-1 forwarding hops, the postOp at the completing step),
 *        "The double binary tree" (bit-trick tree, 14-rank picture).
 *  [FSDP] "FSDP collectives 101", rakshithvasudev.github.io: sections
 *        "All-gather: everyone shows their piece", "Why backward needs a
 *        different collective" (reduce-scatter ownership, avg),
 *        bf16 accumulating in bf16 along the way.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *  - chunk c is finished and owned by rank c; its chain starts at rank c+1
 *    and visits c+2, ..., c (indices mod n);
 *  - the incoming partial is the left operand: acc = incoming (+) own;
 *  - min(a,b) = (b < a) ? b : a, max(a,b) = (b > a) ? b : a;
 *  - float avg multiplies every contribution by s = fp32(1/n) as it is read;
 *    integer avg divides the finished (wrapped) sum once, truncating toward 0;
 *  - bf16/fp16: one hop's arithmetic is done in fp32 and the value that
 *    leaves the hop is rounded to the storage type (round to nearest even);
 *  - all-reduce chunks are cut in 16-byte units,
 *    chunk c = [u*floor(c*V/n), u*floor((c+1)*V/n)) clamped to count, where
 *    u = 16/elem_size and V = ceil(count/u); reduce-scatter and all-gather
 *    use the equal split of their per-rank piece size;
 *  - the tree: parent(v) = (v ^ b) | (b << 1) with b the lowest set bit of v,
 *    falling back to v ^ b when that is >= n; own value first, then the
 *    children's partials in ascending rank order; the root applies the
 *    integer-avg postOp and every rank receives the root's value;
 *  - the double binary tree's second tree mirrors the first (n even) or
 *    shifts it by +1 rank (n odd); the first u*floor(V/2) elements go up the
 *    first tree, the rest up the second;
 *  - the fused pass that combines all ranks at once uses the aligned binary
 *    tree over rank indices (split at the largest power of two below the
 *    range length), lower ranks on the left.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- codes used by this oracle (its own numbering; the Python wrapper maps
 *      names to these) ---- */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2, ORC_I32 = 3 };
enum { ORC_SUM = 0, ORC_PROD = 1, ORC_MIN = 2, ORC_MAX = 3, ORC_AVG = 4 };
enum { ORC_OK = 0, ORC_EBADARG = 1, ORC_ENOMEM = 2 };

/* A value travelling on a wire: fp32 holding a number exactly representable
 * in the storage type, or the 32 bits of an int32. */
typedef union {
    float f;
    uint32_t u;
} val_t;

/* ------------------------------------------------------------------------ */
/* Storage-type conversions, written from the IEEE 754 formats.            */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 is the top half of a binary32. */
static float bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even. */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u = f32_to_bits(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);          /* NaN stays NaN (quiet) */
    uint32_t lower = u & 0xffffu;                          /* the 16 dropped bits   */
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;                                       /* may carry into exponent: correct (overflow to inf) */
    return (uint16_t)upper;
}

/* binary16 -> binary32 (exact). */
static float f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t exp = (h >> 10) & 0x1fu;
    uint32_t man = h & 0x3ffu;
    if (exp == 0x1fu)                                      /* inf / NaN */
        return bits_to_f32(sign | 0x7f800000u | (man << 13));
    if (exp == 0) {
        if (man == 0) return bits_to_f32(sign);            /* +-0 */
        /* subnormal: man * 2^-24, exact in binary32 */
        float v = (float)man * (1.0f / 16777216.0f);
        return sign ? -v : v;
    }
    return bits_to_f32(sign | ((exp - 15u + 127u) << 23) | (man << 13));
}

/* binary32 -> binary16, round to nearest, ties to even. */
static uint16_t f32_to_f16(float f)
{
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t exp = (u >> 23) & 0xffu;
    uint32_t man = u & 0x7fffffu;
    if (exp == 0xffu)                                      /* inf / NaN */
        return (uint16_t)(sign | 0x7c00u | (man ? 0x200u : 0u));
    int e = (int)exp - 127;                                /* unbiased exponent */
    if (e > 15)
        return (uint16_t)(sign | 0x7c00u);                 /* overflow -> inf */
    /* significand with the hidden bit, 24 bits (binary32 subnormals have none
     * and are far below the binary16 range, so they round to zero below) */
    uint32_t sig = exp ? (man | 0x800000u) : man;
    int shift;                                             /* bits to drop from sig */
    uint32_t hexp;                                         /* biased binary16 exponent */
    if (e >= -14) { shift = 13; hexp = (uint32_t)(e + 15); }
    else {                                                 /* binary16 subnormal range */
        shift = 13 + (-14 - e);
        hexp = 0;
        if (shift > 24 + 1) return sign;                   /* far below half the smallest subnormal */
    }
    uint32_t kept = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (kept & 1u))) kept += 1u;
    if (hexp) {
        /* kept holds 11 bits (hidden bit included); a carry to 12 bits bumps the exponent */
        uint32_t r = ((hexp << 10) + (kept - 0x400u));
        if (kept == 0x800u) r = (hexp + 1u) << 10;
        if (r >= 0x7c00u) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | r);
    }
    /* subnormal: kept is the 10-bit mantissa; a carry to 0x400 is the smallest normal */
    return (uint16_t)(sign | kept);
}

/* Exported so the tests can pin the conversions against library routines. */
uint16_t orc_f32_to_bf16(float f) { return f32_to_bf16(f); }
float orc_bf16_to_f32(uint16_t h) { return bf16_to_f32(h); }
uint16_t orc_f32_to_f16(float f) { return f32_to_f16(f); }
float orc_f16_to_f32(uint16_t h) { return f16_to_f32(h); }

/* ------------------------------------------------------------------------ */
/* Element access and the reduction operator.                               */
/* ------------------------------------------------------------------------ */

static size_t elem_size(int dtype) { return (dtype == ORC_F32 || dtype == ORC_I32) ? 4 : 2; }

static val_t load_elem(int dtype, const void *buf, size_t i)
{
    val_t v;
    switch (dtype) {
    case ORC_F32: v.f = ((const float *)buf)[i]; break;
    case ORC_BF16: v.f = bf16_to_f32(((const uint16_t *)buf)[i]); break;
    case ORC_F16: v.f = f16_to_f32(((const uint16_t *)buf)[i]); break;
    default: v.u = ((const uint32_t *)buf)[i]; break;
    }
    return v;
}

/* v must already be representable in the storage type (see round_to_type). */
static void store_elem(int dtype, void *buf, size_t i, val_t v)
{
    switch (dtype) {
    case ORC_F32: ((float *)buf)[i] = v.f; break;
    case ORC_BF16: ((uint16_t *)buf)[i] = f32_to_bf16(v.f); break;
    case ORC_F16: ((uint16_t *)buf)[i] = f32_to_f16(v.f); break;
    default: ((uint32_t *)buf)[i] = v.u; break;
    }
}

/* Round an fp32 result to the storage type, the way a value leaves a hop. */
static val_t round_to_type(int dtype, val_t v)
{
    if (dtype == ORC_BF16) v.f = bf16_to_f32(f32_to_bf16(v.f));
    else if (dtype == ORC_F16) v.f = f16_to_f32(f32_to_f16(v.f));
    return v;
}

/* The contribution as it is read: float avg pre-scales by s = fp32(1/n). */
static val_t pre_op(int dtype, int op, val_t own, float s)
{
    if (op == ORC_AVG && dtype != ORC_I32) own.f = own.f * s;
    return own;
}

/* acc (+) own, computed in fp32 for the float types and in 32-bit two's
 * complement for int32 (sum and prod wrap modulo 2^32). */
static val_t combine(int dtype, int op, val_t acc, val_t own)
{
    val_t r;
    if (dtype == ORC_I32) {
        int32_t a = (int32_t)acc.u, b = (int32_t)own.u;
        switch (op) {
        case ORC_SUM: case ORC_AVG: r.u = acc.u + own.u; break;
        case ORC_PROD: r.u = acc.u * own.u; break;
        case ORC_MIN: r.u = (uint32_t)((b < a) ? b : a); break;
        default: r.u = (uint32_t)((b > a) ? b : a); break;
        }
        return r;
    }
    switch (op) {
    case ORC_SUM: case ORC_AVG: r.f = acc.f + own.f; break;
    case ORC_PROD: r.f = acc.f * own.f; break;
    case ORC_MIN: r.f = (own.f < acc.f) ? own.f : acc.f; break;
    default: r.f = (own.f > acc.f) ? own.f : acc.f; break;
    }
    return r;
}

/* The fixup at the step where a chunk completes: integer avg divides the
 * finished sum by n once (C division, truncating toward zero). */
static val_t post_op(int dtype, int op, int n, val_t acc)
{
    if (op == ORC_AVG && dtype == ORC_I32) acc.u = (uint32_t)((int32_t)acc.u / (int32_t)n);
    return acc;
}

/* ------------------------------------------------------------------------ */
/* Numerics variants: the two accuracy trades the pages name ("FSDP          */
/* collectives 101": bf16 reductions accumulate in bf16 along the way, which */
/* grows lossy with the world size, hence reducing in fp32; fp16 averages    */
/* split the divisor across pre- and post-scaling to avoid overflow).        */
/*   acc32:     bf16 / fp16 partials stay in fp32 between hops; the result   */
/*              is rounded to the storage type once, where it completes.     */
/*   avg_split: float avg pre-scales by 1/p as read, p = 2^e with e the      */
/*              least integer such that 4^e >= n (p near sqrt(n), a power of */
/*              two so the pre-scale is exact), and divides the finished sum */
/*              by q = n/p (the value of p is a reading: the pages give none).*/
/* The defaults (both 0) are the behaviour described everywhere above.       */
/* ------------------------------------------------------------------------ */
typedef struct {
    int acc32;
    int avg_split;
} numerics_t;


static int split_p(int n)
{
    int p = 1;
    while (p * p < n) p *= 2;                               /* 4^e >= n  <=>  (2^e)^2 >= n */
    return p;
}

/* The avg pre-scale of every floating-point contribution. */
static float avg_scale(int n, const numerics_t *nm)
{
    return nm->avg_split ? (float)(1.0 / (double)split_p(n)) : (float)(1.0 / (double)n);
}

/* A partial as it leaves a hop. */
static val_t round_partial(int dtype, val_t v, const numerics_t *nm)
{
    return nm->acc32 ? v : round_to_type(dtype, v);
}

/* Where a reduction completes: the postOp, the split avg's post-division
 * (an fp32 division), and the rounding to the storage type. */
static val_t finish(int dtype, int op, int n, val_t v, const numerics_t *nm)
{
    v = post_op(dtype, op, n, v);
    if (op == ORC_AVG && dtype != ORC_I32 && nm->avg_split) v.f = v.f / (float)((double)n / split_p(n));
    return round_to_type(dtype, v);
}

static int bad_args(int dtype, int op, int n)
{
    return dtype < ORC_F32 || dtype > ORC_I32 || op < ORC_SUM || op > ORC_AVG || n < 1;
}

static int mod_n(long long a, int n) { long long m = a % n; return (int)(m < 0 ? m + n : m); }

/* ------------------------------------------------------------------------ */
/* Counters: one transfer of one chunk from one rank to its ring successor   */
/* is one hop.                                                               */
/* ------------------------------------------------------------------------ */
typedef struct {
    long long *hops_per_chunk;   /* [n] or NULL */
    long long *bytes_sent;       /* [n] per sending rank, or NULL */
} counters_t;

static void count_send(counters_t *k, int rank, int chunk, size_t bytes)
{
    if (k->hops_per_chunk) k->hops_per_chunk[chunk] += 1;
    if (k->bytes_sent) k->bytes_sent[rank] += (long long)bytes;
}

/* ------------------------------------------------------------------------ */
/* The ring, reduce-scatter half.                                            */
/*                                                                           */
/* Chunk c lives at [off[c], off[c+1]) of every rank's input.  At ring step  */
/* t = 0..n-2 every rank r sends the running total of chunk (r-1-t) mod n to */
/* rank r+1: at t = 0 that is its own contribution alone ("send"), later it  */
/* is what it received at t-1 combined with its own ("recvReduceSend").      */
/* Then every rank r receives chunk r, adds its own contribution, and the    */
/* chunk is complete there ("recvReduceCopySend" with the postOp); the       */
/* finished chunk is left in fin[r].                                         */
/* ------------------------------------------------------------------------ */
static int ring_reduce_phase(int dtype, int op, int n, const size_t *off,
                             const void *const *x, val_t **fin, counters_t *k, const numerics_t *nm)
{
    const float s = avg_scale(n, nm);
    size_t maxlen = 0;
    for (int c = 0; c < n; ++c)
        if (off[c + 1] - off[c] > maxlen) maxlen = off[c + 1] - off[c];
    size_t esz = elem_size(dtype);

    /* wire[r]: the message rank r is sending this step; inbox[r]: the message
     * rank r received at the previous step. */
    val_t **wire = calloc((size_t)n, sizeof(val_t *));
    val_t **inbox = calloc((size_t)n, sizeof(val_t *));
    if (!wire || !inbox) { free(wire); free(inbox); return ORC_ENOMEM; }
    int rc = ORC_OK;
    for (int r = 0; r < n; ++r) {
        wire[r] = malloc((maxlen ? maxlen : 1) * sizeof(val_t));
        inbox[r] = malloc((maxlen ? maxlen : 1) * sizeof(val_t));
        if (!wire[r] || !inbox[r]) rc = ORC_ENOMEM;
    }
    if (rc != ORC_OK) goto done;

    for (int t = 0; t <= n - 2; ++t) {
        for (int r = 0; r < n; ++r) {
            int c = mod_n((long long)r - 1 - t, n);
            size_t len = off[c + 1] - off[c];
            const void *mine = x[r];
            val_t *msg = wire[r];
            val_t *in = inbox[r];
            long long i;
#pragma omp parallel for schedule(static)
            for (i = 0; i < (long long)len; ++i) {
                val_t own = pre_op(dtype, op, load_elem(dtype, mine, off[c] + (size_t)i), s);
                msg[i] = (t == 0) ? round_partial(dtype, own, nm)
                                  : round_partial(dtype, combine(dtype, op, in[i], own), nm);
            }
            count_send(k, r, c, len * esz);
        }
        /* deliver: rank r+1's inbox receives rank r's message */
        for (int r = 0; r < n; ++r) {
            int to = (r + 1) % n;
            val_t *tmp = inbox[to];
            inbox[to] = wire[r];
            wire[r] = tmp;
        }
    }

    /* completing step: rank r receives chunk r and finishes it */
    for (int r = 0; r < n; ++r) {
        int c = r;
        size_t len = off[c + 1] - off[c];
        const void *mine = x[r];
        val_t *in = inbox[r];
        val_t *out = fin[r];
        long long i;
#pragma omp parallel for schedule(static)
        for (i = 0; i < (long long)len; ++i) {
            val_t own = pre_op(dtype, op, load_elem(dtype, mine, off[c] + (size_t)i), s);
            val_t v = (n == 1) ? round_partial(dtype, own, nm)
                               : round_partial(dtype, combine(dtype, op, in[i], own), nm);
            out[i] = finish(dtype, op, n, v, nm);
        }
    }

done:
    for (int r = 0; r < n; ++r) { free(wire[r]); free(inbox[r]); }
    free(wire);
    free(inbox);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* The ring, all-gather half.  Every rank r holds finished chunk r in fin[r] */
/* and keeps it (writes it to its own output).  At step t = 0..n-2 rank r    */
/* forwards chunk (r-t) mod n to rank r+1, which stores it and forwards it   */
/* at the next step ("recvCopySend"; the last step is a plain "recv").       */
/* ------------------------------------------------------------------------ */
static int ring_gather_phase(int dtype, int n, const size_t *off, val_t **fin,
                             void *const *y, counters_t *k)
{
    size_t esz = elem_size(dtype);
    size_t maxlen = 0;
    for (int c = 0; c < n; ++c)
        if (off[c + 1] - off[c] > maxlen) maxlen = off[c + 1] - off[c];
    val_t **hold = calloc((size_t)n, sizeof(val_t *));   /* what rank r forwards next */
    val_t **recv = calloc((size_t)n, sizeof(val_t *));
    if (!hold || !recv) { free(hold); free(recv); return ORC_ENOMEM; }
    int rc = ORC_OK;
    for (int r = 0; r < n; ++r) {
        hold[r] = malloc((maxlen ? maxlen : 1) * sizeof(val_t));
        recv[r] = malloc((maxlen ? maxlen : 1) * sizeof(val_t));
        if (!hold[r] || !recv[r]) rc = ORC_ENOMEM;
    }
    if (rc != ORC_OK) goto done;

    /* keep: rank r writes its own finished chunk */
    for (int r = 0; r < n; ++r) {
        size_t len = off[r + 1] - off[r];
        for (size_t i = 0; i < len; ++i) {
            store_elem(dtype, y[r], off[r] + i, fin[r][i]);
            hold[r][i] = fin[r][i];
        }
    }
    for (int t = 0; t <= n - 2; ++t) {
        for (int r = 0; r < n; ++r) {
            int c = mod_n((long long)r - t, n);
            int to = (r + 1) % n;
            size_t len = off[c + 1] - off[c];
            memcpy(recv[to], hold[r], len * sizeof(val_t));
            count_send(k, r, c, len * esz);
        }
        for (int r = 0; r < n; ++r) {
            int c = mod_n((long long)r - 1 - t, n);       /* chunk rank r just received */
            size_t len = off[c + 1] - off[c];
            for (size_t i = 0; i < len; ++i) store_elem(dtype, y[r], off[c] + i, recv[r][i]);
            val_t *tmp = hold[r];
            hold[r] = recv[r];
            recv[r] = tmp;
        }
    }

done:
    for (int r = 0; r < n; ++r) { free(hold[r]); free(recv[r]); }
    free(hold);
    free(recv);
    return rc;
}

static int alloc_fin(int n, const size_t *off, val_t ***fin_out)
{
    val_t **fin = calloc((size_t)n, sizeof(val_t *));
    if (!fin) return ORC_ENOMEM;
    for (int r = 0; r < n; ++r) {
        size_t len = off[r + 1] - off[r];
        fin[r] = malloc((len ? len : 1) * sizeof(val_t));
        if (!fin[r]) {
            for (int q = 0; q < r; ++q) free(fin[q]);
            free(fin);
            return ORC_ENOMEM;
        }
    }
    *fin_out = fin;
    return ORC_OK;
}

static void free_fin(int n, val_t **fin)
{
    if (!fin) return;
    for (int r = 0; r < n; ++r) free(fin[r]);
    free(fin);
}

/* All-reduce chunk bounds, cut in 16-byte units (see the header comment). */
void orc_allreduce_chunks(int dtype, int n, size_t count, size_t *off /* [n+1] */)
{
    size_t u = 16 / elem_size(dtype);
    size_t V = (count + u - 1) / u;
    for (int c = 0; c <= n; ++c) {
        size_t b = u * (size_t)(((unsigned __int128)c * V) / (unsigned)n);
        off[c] = b < count ? b : count;
    }
}

/* Ring all-reduce: y_r[i] for every rank r = the chunk's ring reduction.
 * In place (x[r] == y[r]) is allowed.  hops/bytes may be NULL. */
int orc_ring_allreduce_ex(int dtype, int op, int n, size_t count, const void *const *x,
                          void *const *y, long long *hops_per_chunk, long long *bytes_sent, int acc32, int avg_split)
{
    if (bad_args(dtype, op, n)) return ORC_EBADARG;
    const numerics_t nm = {acc32, avg_split};
    size_t *off = malloc(((size_t)n + 1) * sizeof(size_t));
    if (!off) return ORC_ENOMEM;
    orc_allreduce_chunks(dtype, n, count, off);
    counters_t k = {hops_per_chunk, bytes_sent};
    val_t **fin = NULL;
    int rc = alloc_fin(n, off, &fin);
    if (rc == ORC_OK) rc = ring_reduce_phase(dtype, op, n, off, x, fin, &k, &nm);
    if (rc == ORC_OK) rc = ring_gather_phase(dtype, n, off, fin, y, &k);
    free_fin(n, fin);
    free(off);
    return rc;
}

int orc_ring_allreduce(int dtype, int op, int n, size_t count, const void *const *x,
                       void *const *y, long long *hops_per_chunk, long long *bytes_sent)
{
    return orc_ring_allreduce_ex(dtype, op, n, count, x, y, hops_per_chunk, bytes_sent, 0, 0);
}

/* Ring reduce-scatter: every rank contributes n*recvcount elements; rank r
 * receives the finished chunk r = elements [r*recvcount, (r+1)*recvcount). */
int orc_ring_reduce_scatter_ex(int dtype, int op, int n, size_t recvcount, const void *const *x,
                               void *const *y, long long *hops_per_chunk, long long *bytes_sent, int acc32,
                               int avg_split)
{
    if (bad_args(dtype, op, n)) return ORC_EBADARG;
    const numerics_t nm = {acc32, avg_split};
    size_t *off = malloc(((size_t)n + 1) * sizeof(size_t));
    if (!off) return ORC_ENOMEM;
    for (int c = 0; c <= n; ++c) off[c] = (size_t)c * recvcount;
    counters_t k = {hops_per_chunk, bytes_sent};
    val_t **fin = NULL;
    int rc = alloc_fin(n, off, &fin);
    if (rc == ORC_OK) rc = ring_reduce_phase(dtype, op, n, off, x, fin, &k, &nm);
    if (rc == ORC_OK)
        for (int r = 0; r < n; ++r)
            for (size_t i = 0; i < recvcount; ++i) store_elem(dtype, y[r], i, fin[r][i]);
    free_fin(n, fin);
    free(off);
    return rc;
}

int orc_ring_reduce_scatter(int dtype, int op, int n, size_t recvcount, const void *const *x,
                            void *const *y, long long *hops_per_chunk, long long *bytes_sent)
{
    return orc_ring_reduce_scatter_ex(dtype, op, n, recvcount, x, y, hops_per_chunk, bytes_sent, 0, 0);
}

/* Ring all-gather: rank r contributes sendcount elements; every rank
 * receives the concatenation x_0 || x_1 || ... || x_{n-1}.  Bit copies. */
int orc_ring_all_gather(int dtype, int n, size_t sendcount, const void *const *x,
                        void *const *y, long long *hops_per_chunk, long long *bytes_sent)
{
    if (bad_args(dtype, ORC_SUM, n)) return ORC_EBADARG;
    size_t *off = malloc(((size_t)n + 1) * sizeof(size_t));
    if (!off) return ORC_ENOMEM;
    for (int c = 0; c <= n; ++c) off[c] = (size_t)c * sendcount;
    counters_t k = {hops_per_chunk, bytes_sent};
    val_t **fin = NULL;
    int rc = alloc_fin(n, off, &fin);
    if (rc == ORC_OK) {
        for (int r = 0; r < n; ++r)
            for (size_t i = 0; i < sendcount; ++i) fin[r][i] = load_elem(dtype, x[r], i);
        rc = ring_gather_phase(dtype, n, off, fin, y, &k);
    }
    free_fin(n, fin);
    free(off);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* The bit-trick binary tree over n ranks.                                   */
/* ------------------------------------------------------------------------ */
int orc_tree_parent(int n, int v)
{
    if (v <= 0 || v >= n) return -1;                       /* rank 0 is the root */
    int b = v & -v;                                        /* lowest set bit: fixes the depth */
    int p = (v ^ b) | (b << 1);                            /* clear it, set the next bit up */
    if (p >= n) p = v ^ b;                                 /* fallback at the edge of the range */
    return p;
}

/* The second tree of the double binary tree ("The double binary tree": the
 * roles swapped so that the first tree's leaves work as interior nodes): the
 * mirror image of the first when n is even (rank v plays the part of rank
 * n-1-v), the first shifted by one rank when n is odd (rank v plays the part
 * of rank v-1 mod n; the shift direction is a reading).  which = 0 is the
 * first tree itself.  Returns -1 for the root and for v outside [0, n). */
int orc_dtree_parent(int n, int which, int v)
{
    if (v < 0 || v >= n) return -1;
    if (which == 0) return orc_tree_parent(n, v);
    if (n % 2 == 0) {
        int p = orc_tree_parent(n, n - 1 - v);
        return p < 0 ? -1 : n - 1 - p;
    }
    int p = orc_tree_parent(n, (v - 1 + n) % n);
    return p < 0 ? -1 : (p + 1) % n;
}

/* Up phase, for one element: own value first, then each child's partial in
 * ascending rank order. */
static val_t tree_partial_of(int dtype, int op, int n, int which, int v, const void *const *x, size_t i, float s,
                             const numerics_t *nm)
{
    val_t p = round_partial(dtype, pre_op(dtype, op, load_elem(dtype, x[v], i), s), nm);
    for (int ch = 0; ch < n; ++ch)                       /* children may rank below or above v */
        if (ch != v && orc_dtree_parent(n, which, ch) == v)
            p = round_partial(dtype, combine(dtype, op, p, tree_partial_of(dtype, op, n, which, ch, x, i, s, nm)), nm);
    return p;
}

static int tree_root(int n, int which)
{
    for (int v = 0; v < n; ++v)
        if (orc_dtree_parent(n, which, v) < 0) return v;
    return 0;
}

/* Tree all-reduce: reduce up to rank 0, postOp there, broadcast back down.
 * Every rank ends with the root's value. */
int orc_tree_allreduce_ex(int dtype, int op, int n, size_t count, const void *const *x, void *const *y, int acc32,
                          int avg_split)
{
    if (bad_args(dtype, op, n)) return ORC_EBADARG;
    const numerics_t nm = {acc32, avg_split};
    const float s = avg_scale(n, &nm);
    val_t *root = malloc((count ? count : 1) * sizeof(val_t));
    if (!root) return ORC_ENOMEM;
    long long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (long long)count; ++i)
        root[i] = finish(dtype, op, n, tree_partial_of(dtype, op, n, 0, 0, x, (size_t)i, s, &nm), &nm);
    /* broadcast down (the value is unchanged on the way) */
    for (int v = 0; v < n; ++v)
        for (size_t j = 0; j < count; ++j) store_elem(dtype, y[v], j, root[j]);
    free(root);
    return ORC_OK;
}

int orc_tree_allreduce(int dtype, int op, int n, size_t count, const void *const *x, void *const *y)
{
    return orc_tree_allreduce_ex(dtype, op, n, count, x, y, 0, 0);
}

/* Double binary tree all-reduce: half of every buffer is reduced up (and
 * broadcast down) the first tree, the other half the second ("NCCL then
 * assigns half its channels to each tree").  Reading: the halves are cut in
 * 16-byte units like the ring's chunks with n = 2: elements
 * [0, u*floor(V/2)) go up the first tree and the rest up the second, where
 * u = 16 / element size and V = ceil(count / u).  Each tree reduces as the
 * single tree does (own value first, children in ascending rank order, postOp
 * at its root) and every rank receives its root's value. */
int orc_dtree_allreduce_ex(int dtype, int op, int n, size_t count, const void *const *x, void *const *y, int acc32,
                           int avg_split)
{
    if (bad_args(dtype, op, n)) return ORC_EBADARG;
    const numerics_t nm = {acc32, avg_split};
    const float s = avg_scale(n, &nm);
    const size_t u = 16 / elem_size(dtype);
    const size_t V = (count + u - 1) / u;
    const size_t half = u * (V / 2);
    const int root[2] = {tree_root(n, 0), tree_root(n, 1)};
    val_t *res = malloc((count ? count : 1) * sizeof(val_t));
    if (!res) return ORC_ENOMEM;
    long long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (long long)count; ++i) {
        const int which = (size_t)i < half ? 0 : 1;
        res[i] = finish(dtype, op, n, tree_partial_of(dtype, op, n, which, root[which], x, (size_t)i, s, &nm), &nm);
    }
    for (int v = 0; v < n; ++v)
        for (size_t j = 0; j < count; ++j) store_elem(dtype, y[v], j, res[j]);
    free(res);
    return ORC_OK;
}

int orc_dtree_allreduce(int dtype, int op, int n, size_t count, const void *const *x, void *const *y)
{
    return orc_dtree_allreduce_ex(dtype, op, n, count, x, y, 0, 0);
}

/* ------------------------------------------------------------------------ */
/* The plain definition, y = x_0 (+) x_1 (+) ... (+) x_{n-1} in rank order,   */
/* then the avg rule.  For int32 (sum / prod wrap modulo 2^32, which is       */
/* associative and commutative) and for min / max this is exactly what every */
/* schedule computes, whatever its order ("What all-reduce promises": the     */
/* buffers are combined element-wise and every rank gets the same result).   */
/* It reads element i of every rank at offset i, so it can be applied to      */
/* any slice of the buffers.  Only int32 of any op, or min / max of any      */
/* dtype, are accepted.                                                      */
/* ------------------------------------------------------------------------ */
int orc_direct_reduce(int dtype, int op, int n, size_t count, const void *const *x, void *y)
{
    if (bad_args(dtype, op, n)) return ORC_EBADARG;
    if (dtype != ORC_I32 && op != ORC_MIN && op != ORC_MAX) return ORC_EBADARG;
    long long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (long long)count; ++i) {
        val_t acc = load_elem(dtype, x[0], (size_t)i);
        for (int r = 1; r < n; ++r) acc = combine(dtype, op, acc, load_elem(dtype, x[r], (size_t)i));
        store_elem(dtype, y, (size_t)i, post_op(dtype, op, n, acc));
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* The fused pass with all ranks combined at once: the model is the switch   */
/* that sums in transit ("NCCL all-reduce", section "When the switch does     */
/* the math": one load returns the value combined over every rank, one store  */
/* lands it on every rank), whose order of additions the post leaves open.    */
/* Reading: a fixed pairwise order, the aligned binary tree over the rank    */
/* indices.  Ranks [lo, lo+len) combine as [lo, lo+h) (+) [lo+h, lo+len),    */
/* h the largest power of two below len; the lower ranks are the left        */
/* operand (so min / max ties keep them).  A rank's contribution enters as a */
/* storage-type value (float avg pre-scales it by s = fp32(1/n) first), every */
/* combine is computed in fp32 (int32: wrapping) and rounded to the storage   */
/* type, and integer avg divides the finished total by n once.  Reads element */
/* i of every rank at offset i, so it applies to any slice of the buffers;    */
/* writes one output array (every rank receives the same values).            */
/* ------------------------------------------------------------------------ */
static val_t pairwise_partial(int dtype, int op, int lo, int len, const void *const *x, size_t i, float s,
                              const numerics_t *nm)
{
    if (len == 1) return round_partial(dtype, pre_op(dtype, op, load_elem(dtype, x[lo], i), s), nm);
    int h = 1;
    while (2 * h < len) h *= 2;                            /* largest power of two below len */
    val_t left = pairwise_partial(dtype, op, lo, h, x, i, s, nm);
    val_t right = pairwise_partial(dtype, op, lo + h, len - h, x, i, s, nm);
    return round_partial(dtype, combine(dtype, op, left, right), nm);
}

int orc_pairwise_reduce_ex(int dtype, int op, int n, size_t count, const void *const *x, void *y, int acc32,
                           int avg_split)
{
    if (bad_args(dtype, op, n)) return ORC_EBADARG;
    const numerics_t nm = {acc32, avg_split};
    const float s = avg_scale(n, &nm);
    long long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (long long)count; ++i)
        store_elem(dtype, y, (size_t)i, finish(dtype, op, n, pairwise_partial(dtype, op, 0, n, x, (size_t)i, s, &nm), &nm));
    return ORC_OK;
}

int orc_pairwise_reduce(int dtype, int op, int n, size_t count, const void *const *x, void *y)
{
    return orc_pairwise_reduce_ex(dtype, op, n, count, x, y, 0, 0);
}

int orc_split_p(int n) { return split_p(n); }

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing at one core); results do not depend on it. */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
