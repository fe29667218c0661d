/*
 * hc_oracle.c -- plain, single-threaded CPU oracle for the emulated ring
 * AllReduce data path and the lossless bf16 exponent codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library: every rule below is written out again here from the sources.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no -ffast-math, no FTZ/DAZ),
 * so that every float add is one IEEE-754 binary32 add, round to nearest even,
 * with subnormals kept.
 *
 * Sources (the text of these pages is the authority):
 *  [CoCoNet]  "Breaking the computation and communication abstraction barrier
 *             in distributed machine learning workloads", section "The idea":
 *             AllReduce is a ReduceScatter (each rank keeps its 1/N slice of
 *             the sum) followed by an AllGather (every rank ends with every
 *             slice); distribution layouts local -> sliced -> replicated.
 *             The same section's fusion example: an AllReduce of gradients
 *             followed by an elementwise optimizer update becomes a
 *             ReduceScatter, the update on each rank's slice, and an
 *             AllGather of the updated slices.
 *  [Overlap]  "Communication-computation overlap", TP case study: the
 *             identity AllReduce = AllGather o ReduceScatter; DDP case study:
 *             a ring moves about twice the buffer per rank.
 *  [ResCCL]   "ResCCL: Resource-Efficient Scheduling for Collective
 *             Communication", section 1 (terms: primitives send, recv,
 *             recvReduceCopy; a chunk is about 1% of the data; a micro-batch
 *             is one execution of the algorithm) and section 3 (Transfer(src,
 *             dst, step, chunkId, opType) tasks; data dependencies exist only
 *             within one chunk).
 *  [CCCL]     "CCCL: In-GPU Compression-Coupled Collective Communication",
 *             section 4.1 (sign and fraction sent raw, the 8-bit bf16 exponent
 *             coded from a frequency table), 4.3 (a local table per thread
 *             block, fixed-length codes), 4.4 (one write round into a
 *             preallocated region), section 5 "Handling data alignment"
 *             (only aligned regions are compressed, the remainder is sent
 *             uncompressed) and "Selective compression" (compress what is
 *             sent, decompress what is received).
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes of the repository):
 *  - Ring indexing: at reduce-scatter step s (0..R-2) receiver q gets slice
 *    (q-2-s) mod R from sender q-1; at all-gather step s receiver q gets slice
 *    (q-1-s) mod R from q-1.  Rank r ends owning slice r.  So element i of
 *    slice j is the left fold hop(...hop(hop(x[j+1], x[j+2]), x[j+3])..., x[j])
 *    over ranks taken in ring order, starting at rank j+1, ending at j.
 *  - bf16 sums: every hop converts both bf16 operands to fp32 exactly, adds
 *    once in fp32 and rounds the sum to bf16, nearest-even (the hop payload is
 *    bf16, as it is on the wire).
 *  - A NaN produced by a hop is returned as the canonical quiet NaN
 *    (0x7FC00000 in fp32, 0x7FC0 in bf16): IEEE-754 does not fix the sign or
 *    payload of a NaN result, so both sides agree on one.
 *  - Chunk = round_up(ceil(N/100), A) elements, A = 1024 (uncompressed) or
 *    16384 (compressed, one codec block).  Chunking never changes a value.
 *  - Fused SGD update: with g the allreduce sum of the gradients (the fold
 *    above) and w the owner's weight, the new weight is w - lr*g with the
 *    product and the difference each rounded once in fp32 (no fused
 *    multiply-add); in bf16 w and g are widened exactly and the difference is
 *    rounded to bf16 nearest-even; a NaN result is the canonical quiet NaN.
 *    The slice owner is rank j for slice j (where the reduce-scatter leaves
 *    the sum); every rank ends with the owners' updated slices.
 *  - The codec byte format "HCZ1" (fixed-length dictionary codes plus an
 *    escape for the exponent, raw sign/mantissa byte) is defined in full
 *    above or_compress below.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

/* Status codes, same numbering as the library's public header documents. */
enum { OR_OK = 0, OR_INVALID = 1, OR_UNSUPPORTED = 2, OR_CAPACITY = 3, OR_CORRUPT = 4 };
enum { OR_F32 = 0, OR_BF16 = 1 };

/* ------------------------------------------------------------------------ */
/* Scalar number formats                                                     */
/* ------------------------------------------------------------------------ */

static float f32_of_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the upper half of an fp32 word, so widening is exact. */
float or_bf16_to_f32(uint16_t h) { return f32_of_bits((uint32_t)h << 16); }

/*
 * Nearest bf16 to the fp32 value with bits u, ties to the even significand
 * (IEEE-754 roundTiesToEven with an 8-bit significand and the fp32 exponent
 * range).  Written from the definition: find the two bf16 neighbours of |x|
 * and compare their exact distances in double (both differences are exact).
 * A magnitude at or beyond max_bf16 + half an ulp overflows to infinity, as
 * IEEE rounding does (the neighbour above max_bf16 is taken to be 2^128).
 */
uint16_t or_f32_to_bf16(uint32_t u)
{
    uint32_t sign = u & 0x80000000u;
    uint32_t mag = u & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return 0x7FC0u;                       /* NaN */
    uint32_t lo = mag & 0xFFFF0000u;                              /* toward 0 */
    if (lo == mag) return (uint16_t)((sign | mag) >> 16);          /* exact, incl. inf */
    uint32_t hi = lo + 0x00010000u;                               /* away from 0 */
    double x = (double)f32_of_bits(mag);
    double vlo = (double)f32_of_bits(lo);
    double vhi = (hi == 0x7F800000u) ? ldexp(1.0, 128) : (double)f32_of_bits(hi);
    double dlo = x - vlo;
    double dhi = vhi - x;
    uint32_t pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = ((lo >> 16) & 1u) ? hi : lo;                      /* tie: even */
    return (uint16_t)((sign | pick) >> 16);
}

/* One recvReduceCopy hop on fp32 words: a single IEEE binary32 add. */
uint32_t or_hop_f32(uint32_t a, uint32_t b)
{
    float s = f32_of_bits(a) + f32_of_bits(b);
    if (s != s) return 0x7FC00000u;
    return bits_of_f32(s);
}

/* One recvReduceCopy hop on bf16 words: widen, one fp32 add, round to bf16. */
uint16_t or_hop_bf16(uint16_t a, uint16_t b)
{
    float s = or_bf16_to_f32(a) + or_bf16_to_f32(b);
    return or_f32_to_bf16(bits_of_f32(s));
}

/* Fused SGD update of one weight: w - lr*g, product and difference rounded
 * once each in fp32. */
uint32_t or_sgd_f32(uint32_t w, uint32_t g, float lr)
{
    float t = lr * f32_of_bits(g);
    float r = f32_of_bits(w) - t;
    if (r != r) return 0x7FC00000u;
    return bits_of_f32(r);
}

/* The same on bf16 words: widen w and g, the fp32 steps above, round the
 * result to bf16. */
uint16_t or_sgd_bf16(uint16_t w, uint16_t g, float lr)
{
    float t = lr * or_bf16_to_f32(g);
    float r = or_bf16_to_f32(w) - t;
    return or_f32_to_bf16(bits_of_f32(r));
}

static size_t elem_size(int dtype) { return dtype == OR_F32 ? 4 : 2; }

static uint32_t load_elem(const void *base, size_t i, int dtype)
{
    if (dtype == OR_F32) return ((const uint32_t *)base)[i];
    return ((const uint16_t *)base)[i];
}

static void store_elem(void *base, size_t i, int dtype, uint32_t v)
{
    if (dtype == OR_F32) ((uint32_t *)base)[i] = v;
    else ((uint16_t *)base)[i] = (uint16_t)v;
}

static uint32_t hop(uint32_t a, uint32_t b, int dtype)
{
    if (dtype == OR_F32) return or_hop_f32(a, b);
    return or_hop_bf16((uint16_t)a, (uint16_t)b);
}

static size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }
static size_t round_up(size_t a, size_t b) { return ceil_div(a, b) * b; }
static int mod(int a, int r) { int m = a % r; return m < 0 ? m + r : m; }

/* ------------------------------------------------------------------------ */
/* Ring schedule                                                             */
/* ------------------------------------------------------------------------ */

/* Elements per slice.  Reduce-scatter and all-gather need n % R == 0; an
 * allreduce of any n uses ceil(n/R), so the last slices are short or empty. */
size_t or_slice_len(size_t n, int R) { return ceil_div(n, (size_t)R); }

/* Chunk of roughly 1% of the per-rank buffer, rounded up to the alignment
 * unit (ResCCL section 1: a chunk is about 1% of the data). */
size_t or_chunk_elems(size_t n, size_t align)
{
    size_t c = round_up(ceil_div(n, 100), align);
    return c == 0 ? align : c;
}

/* One task of the ring in ResCCL's Transfer(srcRank, dstRank, step, chunkId,
 * opType) form, with the element range it covers inside the per-rank buffer. */
typedef struct {
    int32_t src, dst, step, chunk;
    int32_t op;          /* 1 = recvReduceCopy (reduce-scatter), 2 = recv/copy (all-gather) */
    int32_t slice;
    uint64_t off, len;   /* element range in the per-rank buffer */
} or_task_t;

enum { OR_OP_RRC = 1, OR_OP_COPY = 2 };

/*
 * Emit the ring allreduce as a task list: R-1 reduce-scatter steps, then R-1
 * all-gather steps; inside a step, receiver-major then chunk order.  Returns
 * the number of tasks; writes at most cap of them (tasks may be NULL to
 * count).  Empty ranges (short tail slices) produce no task.
 */
size_t or_ring_tasks(int R, size_t n, size_t chunk, or_task_t *tasks, size_t cap)
{
    size_t L = or_slice_len(n, R), count = 0;
    for (int phase = 0; phase < 2; ++phase) {
        for (int s = 0; s + 1 < R; ++s) {
            for (int q = 0; q < R; ++q) {
                int p = mod(q - 1, R);
                int j = phase == 0 ? mod(q - 2 - s, R) : mod(q - 1 - s, R);
                size_t lo = (size_t)j * L, hi = lo + L;
                if (lo > n) lo = n;
                if (hi > n) hi = n;
                size_t nchunks = ceil_div(hi - lo, chunk);
                for (size_t c = 0; c < nchunks; ++c) {
                    if (tasks && count < cap) {
                        or_task_t *t = &tasks[count];
                        t->src = p; t->dst = q; t->step = s; t->chunk = (int32_t)c;
                        t->op = phase == 0 ? OR_OP_RRC : OR_OP_COPY;
                        t->slice = j;
                        t->off = lo + c * chunk;
                        t->len = (hi - t->off) < chunk ? (hi - t->off) : chunk;
                    }
                    ++count;
                }
            }
        }
    }
    return count;
}

/*
 * Closed form of the ring allreduce.  Element i of slice j is the left fold
 * over ranks j+1, j+2, ..., j (mod R).  Every rank's output gets a copy of the
 * same words, so all ranks end identical (CoCoNet: local -> replicated).
 */
int or_allreduce_fold(const void *const *x, void *const *out, size_t n, int dtype, int R)
{
    if (R < 1 || (dtype != OR_F32 && dtype != OR_BF16)) return OR_INVALID;
    size_t L = or_slice_len(n, R);
    for (size_t i = 0; i < n; ++i) {
        int j = (int)(i / L);
        uint32_t acc = load_elem(x[mod(j + 1, R)], i, dtype);
        for (int k = 2; k <= R; ++k)
            acc = hop(acc, load_elem(x[mod(j + k, R)], i, dtype), dtype);
        for (int r = 0; r < R; ++r) store_elem(out[r], i, dtype, acc);
    }
    return OR_OK;
}

/*
 * Allreduce of gradients fused with an SGD update (CoCoNet's fusion): g is the
 * fold above; the owner of slice j (rank j) updates its weights there, and
 * every rank's output holds the updated weights.  w_in[r] are the ranks'
 * weights before the call; only the owner's copy of a slice is read.
 */
int or_allreduce_sgd(const void *const *grads, const void *const *w_in, void *const *w_out, size_t n,
                     int dtype, int R, float lr)
{
    if (R < 1 || (dtype != OR_F32 && dtype != OR_BF16)) return OR_INVALID;
    size_t L = or_slice_len(n, R);
    for (size_t i = 0; i < n; ++i) {
        int j = (int)(i / L);
        uint32_t g = load_elem(grads[mod(j + 1, R)], i, dtype);
        for (int k = 2; k <= R; ++k)
            g = hop(g, load_elem(grads[mod(j + k, R)], i, dtype), dtype);
        uint32_t w = load_elem(w_in[j], i, dtype);
        uint32_t nw = dtype == OR_F32 ? or_sgd_f32(w, g, lr) : or_sgd_bf16((uint16_t)w, (uint16_t)g, lr);
        for (int r = 0; r < R; ++r) store_elem(w_out[r], i, dtype, nw);
    }
    return OR_OK;
}

/* The same fold evaluated only at chosen element indices (for sampled checks
 * of large buffers): vals[k] = allreduce result at idx[k]. */
int or_allreduce_fold_at(const void *const *x, size_t n, int dtype, int R,
                         const uint64_t *idx, size_t m, void *vals)
{
    if (R < 1 || (dtype != OR_F32 && dtype != OR_BF16)) return OR_INVALID;
    size_t L = or_slice_len(n, R);
    for (size_t k = 0; k < m; ++k) {
        size_t i = idx[k];
        if (i >= n) return OR_INVALID;
        int j = (int)(i / L);
        uint32_t acc = load_elem(x[mod(j + 1, R)], i, dtype);
        for (int t = 2; t <= R; ++t)
            acc = hop(acc, load_elem(x[mod(j + t, R)], i, dtype), dtype);
        store_elem(vals, k, dtype, acc);
    }
    return OR_OK;
}

/*
 * The fp32-carry reading of "fp32 accumulation, bf16 round-to-nearest-even
 * output" (bf16 data only): the reduce-scatter partials stay in fp32 and the
 * sum is rounded to bf16 once.  Element i of slice j: acc starts as the exact
 * fp32 value of x[j+1][i]; each later rank's value (x[j+2], ..., x[j]) is
 * widened exactly and added with one fp32 add (a NaN sum becomes the
 * canonical fp32 NaN); then out = bf16(acc), nearest even.  With one rank
 * nothing is added and the output is the input, bit for bit.
 */
int or_allreduce_fold_f32carry(const void *const *x, void *const *out, size_t n, int R)
{
    if (R < 1) return OR_INVALID;
    size_t L = or_slice_len(n, R);
    for (size_t i = 0; i < n; ++i) {
        int j = (int)(i / L);
        uint16_t res;
        if (R == 1) {
            res = ((const uint16_t *)x[0])[i];
        } else {
            uint32_t acc = bits_of_f32(or_bf16_to_f32(((const uint16_t *)x[mod(j + 1, R)])[i]));
            for (int k = 2; k <= R; ++k) {
                uint16_t v = ((const uint16_t *)x[mod(j + k, R)])[i];
                acc = or_hop_f32(acc, bits_of_f32(or_bf16_to_f32(v)));
            }
            res = or_f32_to_bf16(acc);
        }
        for (int r = 0; r < R; ++r) ((uint16_t *)out[r])[i] = res;
    }
    return OR_OK;
}

/*
 * Step simulator of the ring allreduce: R explicit output buffers, the task
 * list above executed in order.  At reduce-scatter step 0 the sender's
 * contribution is its input; later it is the partial the sender wrote in its
 * own output buffer at the previous step.  All-gather copies the sender's
 * output slice.  out[r] must not alias x[r].
 */
int or_allreduce_ring(const void *const *x, void *const *out, size_t n, int dtype, int R,
                      size_t chunk)
{
    if (R < 1 || chunk == 0 || (dtype != OR_F32 && dtype != OR_BF16)) return OR_INVALID;
    size_t es = elem_size(dtype);
    if (R == 1) { memcpy(out[0], x[0], n * es); return OR_OK; }
    size_t nt = or_ring_tasks(R, n, chunk, NULL, 0);
    or_task_t *tasks = (or_task_t *)malloc(sizeof(or_task_t) * (nt ? nt : 1));
    if (!tasks) return OR_CAPACITY;
    or_ring_tasks(R, n, chunk, tasks, nt);
    for (size_t k = 0; k < nt; ++k) {
        const or_task_t *t = &tasks[k];
        for (size_t i = t->off; i < t->off + t->len; ++i) {
            if (t->op == OR_OP_RRC) {
                const void *src = t->step == 0 ? x[t->src] : out[t->src];
                uint32_t v = hop(load_elem(src, i, dtype), load_elem(x[t->dst], i, dtype), dtype);
                store_elem(out[t->dst], i, dtype, v);
            } else {
                store_elem(out[t->dst], i, dtype, load_elem(out[t->src], i, dtype));
            }
        }
    }
    free(tasks);
    return OR_OK;
}

/*
 * Reduce-scatter by step simulation.  x[r] holds recvcount*R elements; out[r]
 * receives slice r (recvcount elements).  Partials travel in per-rank scratch
 * buffers, as a receive FIFO would hold them.
 */
int or_reduce_scatter_ring(const void *const *x, void *const *out, size_t recvcount, int dtype,
                           int R, size_t chunk)
{
    if (R < 1 || chunk == 0 || (dtype != OR_F32 && dtype != OR_BF16)) return OR_INVALID;
    size_t es = elem_size(dtype), L = recvcount, n = recvcount * (size_t)R;
    if (R == 1) { memcpy(out[0], x[0], n * es); return OR_OK; }
    /* part[r] holds rank r's latest partial, indexed like the full buffer. */
    void **part = (void **)calloc((size_t)R, sizeof(void *));
    void **next = (void **)calloc((size_t)R, sizeof(void *));
    if (!part || !next) { free(part); free(next); return OR_CAPACITY; }
    for (int r = 0; r < R; ++r) {
        part[r] = calloc(n ? n : 1, es);
        next[r] = calloc(n ? n : 1, es);
    }
    for (int s = 0; s + 1 < R; ++s) {
        for (int q = 0; q < R; ++q) {
            int p = mod(q - 1, R), j = mod(q - 2 - s, R);
            size_t lo = (size_t)j * L;
            for (size_t c0 = 0; c0 < L; c0 += chunk) {
                size_t c1 = c0 + chunk < L ? c0 + chunk : L;
                for (size_t i = lo + c0; i < lo + c1; ++i) {
                    const void *src = s == 0 ? x[p] : part[p];
                    uint32_t v = hop(load_elem(src, i, dtype), load_elem(x[q], i, dtype), dtype);
                    store_elem(next[q], i, dtype, v);
                }
            }
        }
        for (int r = 0; r < R; ++r) { void *t = part[r]; part[r] = next[r]; next[r] = t; }
    }
    for (int r = 0; r < R; ++r)
        memcpy(out[r], (const char *)part[r] + (size_t)r * L * es, L * es);
    for (int r = 0; r < R; ++r) { free(part[r]); free(next[r]); }
    free(part); free(next);
    return OR_OK;
}

/*
 * All-gather by step simulation.  x[r] holds sendcount elements; out[r]
 * receives R*sendcount, slice j = x[j].  Step 0 also places each rank's own
 * contribution in its own output (the local copy).
 */
int or_all_gather_ring(const void *const *x, void *const *out, size_t sendcount, int dtype,
                       int R, size_t chunk)
{
    if (R < 1 || chunk == 0 || (dtype != OR_F32 && dtype != OR_BF16)) return OR_INVALID;
    size_t es = elem_size(dtype), L = sendcount;
    for (int r = 0; r < R; ++r)
        memcpy((char *)out[r] + (size_t)r * L * es, x[r], L * es);
    for (int s = 0; s + 1 < R; ++s) {
        for (int q = 0; q < R; ++q) {
            int p = mod(q - 1, R), j = mod(q - 1 - s, R);
            for (size_t c0 = 0; c0 < L; c0 += chunk) {
                size_t c1 = c0 + chunk < L ? c0 + chunk : L;
                memcpy((char *)out[q] + ((size_t)j * L + c0) * es,
                       (const char *)out[p] + ((size_t)j * L + c0) * es, (c1 - c0) * es);
            }
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* HCZ1: lossless bf16 codec                                                 */
/* ------------------------------------------------------------------------ */
/*
 * Principle (CCCL section 4.1): a bf16 word is sign | 8-bit exponent | 7-bit
 * fraction.  Sign and fraction are near random and are sent raw; the exponent
 * is skewed and is coded.  Each block builds its own frequency table (section
 * 4.3), codes with fixed-length codes (section 4.3), and writes its record in
 * one pass (section 4.4).  Only whole blocks are coded; a partial tail block is
 * stored raw (section 5, "Handling data alignment").
 *
 * Byte format (little-endian; every padding byte is zero):
 *   stream header, 32 bytes:
 *     u32 magic = 0x315A4348 ("HCZ1"), u32 block_elems B (= 16384),
 *     u64 n (elements), u32 n_blocks = ceil(n/B), u32 flags = 0,
 *     u64 total_bytes
 *   u64 rec_off[n_blocks] (byte offset of each record from the stream start),
 *     zero padded to a multiple of 16 bytes
 *   records in block order, back to back, each a multiple of 16 bytes.
 *   record header, 16 bytes: u8 mode (0 raw, 1 coded), u8 b, u16 0,
 *     u32 m (elements in the block), u32 n_esc, u32 rec_bytes
 *   raw record:   the m bf16 words, zero padded to 16.  b = n_esc = 0.
 *   coded record (only when m == B):
 *     dictionary, max(16, 2^b) bytes: the K = 2^b - 1 most frequent exponents,
 *       most frequent first, then zeros
 *     code planes, b planes of B/8 bytes: bit (i mod 8) of byte (i div 8) of
 *       plane k is bit k of code[i]; code[i] = dictionary index of exponent i,
 *       or K (escape) when the exponent is not in the dictionary
 *     sign/mantissa plane, B bytes: sm[i] = (sign << 7) | fraction
 *     escape plane: the exponent bytes of the escaped elements in index
 *       order, n_esc bytes, zero padded to 16
 *     rec_bytes = 16 + max(16, 2^b) + B*b/8 + B + round_up(n_esc, 16)
 * Encoder choices: ranks = exponents by (count descending, exponent
 * ascending), so the ranking is total and zero-count exponents fill the tail;
 * b = the smallest b in 1..7 with the least rec_bytes; raw when that is not
 * below the raw size 16 + 2B.
 */

#define HCZ_MAGIC 0x315A4348u
#define HCZ_B 16384u

static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint32_t v) { for (int k = 0; k < 4; ++k) p[k] = (uint8_t)(v >> (8 * k)); }
static void put_u64(uint8_t *p, uint64_t v) { for (int k = 0; k < 8; ++k) p[k] = (uint8_t)(v >> (8 * k)); }
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t *p) { uint32_t v = 0; for (int k = 3; k >= 0; --k) v = (v << 8) | p[k]; return v; }
static uint64_t get_u64(const uint8_t *p) { uint64_t v = 0; for (int k = 7; k >= 0; --k) v = (v << 8) | p[k]; return v; }

static size_t hcz_header_bytes(size_t n_blocks) { return 32 + round_up(8 * n_blocks, 16); }
static size_t hcz_raw_bytes(size_t m) { return 16 + round_up(2 * m, 16); }
static size_t hcz_dict_bytes(int b) { return (size_t)1 << b < 16 ? 16 : (size_t)1 << b; }
static size_t hcz_coded_bytes(int b, size_t n_esc)
{
    return 16 + hcz_dict_bytes(b) + (size_t)HCZ_B * (size_t)b / 8 + HCZ_B + round_up(n_esc, 16);
}

/* Largest stream the encoder can produce for n elements (every block raw). */
size_t or_compress_bound(size_t n)
{
    size_t nb = ceil_div(n, HCZ_B), total = hcz_header_bytes(nb);
    for (size_t k = 0; k < nb; ++k) {
        size_t m = (k + 1) * HCZ_B <= n ? HCZ_B : n - k * HCZ_B;
        total += hcz_raw_bytes(m);
    }
    return total;
}

static const uint32_t *g_sort_counts;   /* comparator context (single-threaded) */
static int by_count_then_symbol(const void *pa, const void *pb)
{
    int a = *(const int *)pa, b = *(const int *)pb;
    if (g_sort_counts[a] != g_sort_counts[b]) return g_sort_counts[a] > g_sort_counts[b] ? -1 : 1;
    return a - b;
}

/* Per-block encoder decision, exposed for tests: mode, b, n_esc, rec_bytes. */
typedef struct { int32_t mode, b; uint32_t m, n_esc, rec_bytes; } or_block_plan_t;

static void plan_block(const uint16_t *v, size_t m, or_block_plan_t *plan, int order[256])
{
    plan->m = (uint32_t)m;
    plan->mode = 0; plan->b = 0; plan->n_esc = 0;
    plan->rec_bytes = (uint32_t)hcz_raw_bytes(m);
    for (int s = 0; s < 256; ++s) order[s] = s;
    if (m != HCZ_B) return;
    uint32_t hist[256] = {0};
    for (size_t i = 0; i < m; ++i) hist[(v[i] >> 7) & 0xFF]++;
    g_sort_counts = hist;
    qsort(order, 256, sizeof(int), by_count_then_symbol);
    size_t best = 0; int best_b = 0; size_t best_esc = 0;
    for (int b = 1; b <= 7; ++b) {
        size_t K = ((size_t)1 << b) - 1, covered = 0;
        for (size_t k = 0; k < K; ++k) covered += hist[order[k]];
        size_t esc = m - covered, size = hcz_coded_bytes(b, esc);
        if (best_b == 0 || size < best) { best = size; best_b = b; best_esc = esc; }
    }
    if (best < hcz_raw_bytes(m)) {
        plan->mode = 1; plan->b = best_b; plan->n_esc = (uint32_t)best_esc;
        plan->rec_bytes = (uint32_t)best;
    }
}

int or_plan_block(const uint16_t *v, size_t m, or_block_plan_t *plan)
{
    int order[256];
    if (m == 0 || m > HCZ_B) return OR_INVALID;
    plan_block(v, m, plan, order);
    return OR_OK;
}

/* Write one block's record for a decided plan and symbol order into rec
 * (which has room for plan.rec_bytes). */
static void write_record(const uint16_t *v, size_t m, const or_block_plan_t plan, const int order[256],
                         uint8_t *rec)
{
    memset(rec, 0, plan.rec_bytes);
    rec[0] = (uint8_t)plan.mode;
    rec[1] = (uint8_t)plan.b;
    put_u16(rec + 2, 0);
    put_u32(rec + 4, plan.m);
    put_u32(rec + 8, plan.n_esc);
    put_u32(rec + 12, plan.rec_bytes);
    if (plan.mode == 0) {
        for (size_t i = 0; i < m; ++i) put_u16(rec + 16 + 2 * i, v[i]);
        return;
    }
    int b = plan.b;
    uint32_t K = (1u << b) - 1;
    uint32_t rank[256];
    for (int k = 0; k < 256; ++k) rank[order[k]] = (uint32_t)k;
    uint8_t *dict = rec + 16;
    for (uint32_t k = 0; k < K; ++k) dict[k] = (uint8_t)order[k];
    uint8_t *planes = dict + hcz_dict_bytes(b);
    uint8_t *sm = planes + (size_t)HCZ_B * b / 8;
    uint8_t *esc = sm + HCZ_B;
    size_t ne = 0;
    for (size_t i = 0; i < m; ++i) {
        uint32_t e = (v[i] >> 7) & 0xFF;
        uint32_t code = rank[e] < K ? rank[e] : K;
        for (int k = 0; k < b; ++k)
            if ((code >> k) & 1u) planes[(size_t)k * (HCZ_B / 8) + i / 8] |= (uint8_t)(1u << (i % 8));
        sm[i] = (uint8_t)(((v[i] >> 8) & 0x80) | (v[i] & 0x7F));
        if (code == K) esc[ne++] = (uint8_t)e;
    }
}

/* Encode one block into rec with its own table (the HCZ1 rule). */
static void encode_block(const uint16_t *v, size_t m, uint8_t *rec)
{
    or_block_plan_t plan;
    int order[256];
    plan_block(v, m, &plan, order);
    write_record(v, m, plan, order, rec);
}

/*
 * Compress n bf16 words into an HCZ1 stream.  Returns the stream size in
 * bytes, or 0 when cap is smaller than that size.
 */
size_t or_compress(const uint16_t *in, size_t n, uint8_t *out, size_t cap)
{
    size_t nb = ceil_div(n, HCZ_B);
    size_t hdr = hcz_header_bytes(nb), total = hdr;
    or_block_plan_t plan;
    int order[256];
    for (size_t k = 0; k < nb; ++k) {
        size_t m = (k + 1) * HCZ_B <= n ? HCZ_B : n - k * HCZ_B;
        plan_block(in + k * HCZ_B, m, &plan, order);
        total += plan.rec_bytes;
    }
    if (total > cap) return 0;
    memset(out, 0, hdr);
    put_u32(out + 0, HCZ_MAGIC);
    put_u32(out + 4, HCZ_B);
    put_u64(out + 8, (uint64_t)n);
    put_u32(out + 16, (uint32_t)nb);
    put_u32(out + 20, 0);
    put_u64(out + 24, (uint64_t)total);
    size_t off = hdr;
    for (size_t k = 0; k < nb; ++k) {
        size_t m = (k + 1) * HCZ_B <= n ? HCZ_B : n - k * HCZ_B;
        put_u64(out + 32 + 8 * k, (uint64_t)off);
        encode_block(in + k * HCZ_B, m, out + off);
        off += get_u32(out + off + 12);
    }
    return total;
}

/*
 * Table-scope variant (the sample-size question of CCCL section 4.3, and the
 * global-table baseline of section 4.2): one symbol order and one code length
 * b for each group of `group` consecutive full blocks (group = 0: all full
 * blocks of the stream share one table).  The order is (count desc, symbol
 * asc) over the group's summed histogram; b minimizes the sum over the
 * group's full blocks of their coded record sizes (ties: smaller b); a block
 * whose coded record would not be smaller than its raw record is raw, and
 * partial blocks are raw.  Every record still carries its dictionary, so the
 * stream is an ordinary HCZ1 stream.  group = 1 is or_compress exactly.
 * Returns the stream size, or 0 when cap is too small.
 */
size_t or_compress_scoped(const uint16_t *in, size_t n, uint8_t *out, size_t cap, size_t group)
{
    size_t nb = ceil_div(n, HCZ_B), nfull = n / HCZ_B;
    size_t G = group == 0 ? (nfull ? nfull : 1) : group;
    size_t ngroups = nfull ? ceil_div(nfull, G) : 0;
    int (*orders)[256] = (int (*)[256])malloc(sizeof(int[256]) * (ngroups ? ngroups : 1));
    int *bs = (int *)malloc(sizeof(int) * (ngroups ? ngroups : 1));
    or_block_plan_t *plans = (or_block_plan_t *)malloc(sizeof(or_block_plan_t) * (nb ? nb : 1));
    if (!orders || !bs || !plans) { free(orders); free(bs); free(plans); return 0; }
    for (size_t g = 0; g < ngroups; ++g) {
        size_t k0 = g * G, k1 = k0 + G < nfull ? k0 + G : nfull;
        uint32_t hist[256] = {0};
        for (size_t k = k0; k < k1; ++k)
            for (size_t i = 0; i < HCZ_B; ++i) hist[(in[k * HCZ_B + i] >> 7) & 0xFF]++;
        for (int t = 0; t < 256; ++t) orders[g][t] = t;
        g_sort_counts = hist;
        qsort(orders[g], 256, sizeof(int), by_count_then_symbol);
        size_t best = 0;
        int best_b = 0;
        for (int b = 1; b <= 7; ++b) {
            size_t K = ((size_t)1 << b) - 1, sum = 0;
            for (size_t k = k0; k < k1; ++k) {
                uint32_t bh[256] = {0};
                for (size_t i = 0; i < HCZ_B; ++i) bh[(in[k * HCZ_B + i] >> 7) & 0xFF]++;
                size_t covered = 0;
                for (size_t r = 0; r < K; ++r) covered += bh[orders[g][r]];
                sum += hcz_coded_bytes(b, HCZ_B - covered);
            }
            if (best_b == 0 || sum < best) { best = sum; best_b = b; }
        }
        bs[g] = best_b;
    }
    size_t hdr = hcz_header_bytes(nb), total = hdr;
    for (size_t k = 0; k < nb; ++k) {
        size_t m = (k + 1) * HCZ_B <= n ? HCZ_B : n - k * HCZ_B;
        or_block_plan_t *pl = &plans[k];
        pl->m = (uint32_t)m; pl->mode = 0; pl->b = 0; pl->n_esc = 0;
        pl->rec_bytes = (uint32_t)hcz_raw_bytes(m);
        if (m == HCZ_B) {
            size_t g = k / G;
            int b = bs[g];
            size_t K = ((size_t)1 << b) - 1;
            uint32_t bh[256] = {0};
            for (size_t i = 0; i < HCZ_B; ++i) bh[(in[k * HCZ_B + i] >> 7) & 0xFF]++;
            size_t covered = 0;
            for (size_t r = 0; r < K; ++r) covered += bh[orders[g][r]];
            size_t size = hcz_coded_bytes(b, HCZ_B - covered);
            if (size < hcz_raw_bytes(m)) {
                pl->mode = 1; pl->b = b; pl->n_esc = (uint32_t)(HCZ_B - covered); pl->rec_bytes = (uint32_t)size;
            }
        }
        total += pl->rec_bytes;
    }
    if (total > cap) { free(orders); free(bs); free(plans); return 0; }
    memset(out, 0, hdr);
    put_u32(out + 0, HCZ_MAGIC);
    put_u32(out + 4, HCZ_B);
    put_u64(out + 8, (uint64_t)n);
    put_u32(out + 16, (uint32_t)nb);
    put_u32(out + 20, 0);
    put_u64(out + 24, (uint64_t)total);
    size_t off = hdr;
    int identity[256];
    for (int t = 0; t < 256; ++t) identity[t] = t;
    for (size_t k = 0; k < nb; ++k) {
        size_t m = (k + 1) * HCZ_B <= n ? HCZ_B : n - k * HCZ_B;
        put_u64(out + 32 + 8 * k, (uint64_t)off);
        write_record(in + k * HCZ_B, m, plans[k], m == HCZ_B ? orders[k / G] : identity, out + off);
        off += plans[k].rec_bytes;
    }
    free(orders); free(bs); free(plans);
    return total;
}

/*
 * Decompress an HCZ1 stream of in_bytes bytes holding n elements.  Checks
 * every field before it is used; any mismatch returns OR_CORRUPT and leaves
 * out zero filled.
 */
int or_decompress(const uint8_t *in, size_t in_bytes, uint16_t *out, size_t n)
{
    memset(out, 0, n * 2);
    size_t nb = ceil_div(n, HCZ_B), hdr = hcz_header_bytes(nb);
    if (in_bytes < hdr) return OR_CORRUPT;
    if (get_u32(in) != HCZ_MAGIC || get_u32(in + 4) != HCZ_B || get_u64(in + 8) != n ||
        get_u32(in + 16) != nb || get_u32(in + 20) != 0)
        return OR_CORRUPT;
    uint64_t total = get_u64(in + 24);
    if (total > in_bytes || total < hdr) return OR_CORRUPT;
    for (size_t i = 32 + 8 * nb; i < hdr; ++i) if (in[i]) return OR_CORRUPT;
    uint64_t expect = hdr;
    for (size_t k = 0; k < nb; ++k) {
        uint64_t off = get_u64(in + 32 + 8 * k);
        if (off != expect || off + 16 > total) goto corrupt;
        const uint8_t *rec = in + off;
        size_t m = (k + 1) * HCZ_B <= n ? HCZ_B : n - k * HCZ_B;
        uint32_t mode = rec[0], b = rec[1], rm = get_u32(rec + 4);
        uint32_t n_esc = get_u32(rec + 8), rb = get_u32(rec + 12);
        if (get_u16(rec + 2) != 0 || rm != m) goto corrupt;
        if (off + rb > total) goto corrupt;
        uint16_t *dst = out + k * HCZ_B;
        if (mode == 0) {
            if (b != 0 || n_esc != 0 || rb != hcz_raw_bytes(m)) goto corrupt;
            for (size_t i = 0; i < m; ++i) dst[i] = get_u16(rec + 16 + 2 * i);
            for (size_t i = 16 + 2 * m; i < rb; ++i) if (rec[i]) goto corrupt;
        } else if (mode == 1) {
            if (m != HCZ_B || b < 1 || b > 7 || n_esc > HCZ_B || rb != hcz_coded_bytes((int)b, n_esc))
                goto corrupt;
            uint32_t K = (1u << b) - 1;
            const uint8_t *dict = rec + 16;
            const uint8_t *planes = dict + hcz_dict_bytes((int)b);
            const uint8_t *sm = planes + (size_t)HCZ_B * b / 8;
            const uint8_t *esc = sm + HCZ_B;
            for (size_t i = K; i < hcz_dict_bytes((int)b); ++i) if (dict[i]) goto corrupt;
            size_t ne = 0;
            for (size_t i = 0; i < m; ++i) {
                uint32_t code = 0;
                for (uint32_t p = 0; p < b; ++p)
                    code |= (uint32_t)((planes[(size_t)p * (HCZ_B / 8) + i / 8] >> (i % 8)) & 1u) << p;
                uint32_t e;
                if (code == K) {
                    if (ne >= n_esc) goto corrupt;
                    e = esc[ne++];
                } else {
                    e = dict[code];
                }
                dst[i] = (uint16_t)(((uint32_t)(sm[i] & 0x80) << 8) | (e << 7) | (sm[i] & 0x7F));
            }
            if (ne != n_esc) goto corrupt;
            for (size_t i = n_esc; i < round_up(n_esc, 16); ++i) if (esc[i]) goto corrupt;
        } else {
            goto corrupt;
        }
        expect = off + rb;
    }
    if (expect != total) goto corrupt;
    return OR_OK;
corrupt:
    memset(out, 0, n * 2);
    return OR_CORRUPT;
}

/* ------------------------------------------------------------------------ */
/* Compressed ring allreduce                                                 */
/* ------------------------------------------------------------------------ */
/*
 * The ring allreduce above with every hop payload sent as an HCZ1 stream, one
 * stream per (hop, chunk) (CCCL section 5: compress on the sender, decompress
 * on the receiver, reduce in between).  The chunk is aligned to whole codec
 * blocks, so only a slice's last chunk can end in a partial (raw) block.
 * Reduce-scatter: the sender compresses its payload (its input at step 0,
 * else its partial); the receiver decompresses, applies the bf16 hop with its
 * own input.  All-gather: each receiver decompresses the finished slice into
 * its output and forwards the same bytes; the encoder is deterministic and
 * lossless, so compressing the sender's decoded copy again yields exactly the
 * bytes it received, which is how the stream of each hop is rebuilt here.
 * wire_bytes = sum over all streams of their sizes.  Because the codec is
 * lossless the output equals or_allreduce_ring's bf16 result bit for bit.
 */
int or_compressed_allreduce(const uint16_t *const *x, uint16_t *const *out, size_t n, int R,
                            size_t chunk, uint64_t *wire_bytes)
{
    if (R < 1 || chunk == 0 || chunk % HCZ_B != 0) return OR_INVALID;
    uint64_t wire = 0;
    if (R == 1) { memcpy(out[0], x[0], n * 2); if (wire_bytes) *wire_bytes = 0; return OR_OK; }
    size_t L = or_slice_len(n, R);
    size_t cap = or_compress_bound(chunk);
    uint8_t *stream = (uint8_t *)malloc(cap);
    uint16_t *payload = (uint16_t *)malloc(chunk * 2);
    uint16_t *recv = (uint16_t *)malloc(chunk * 2);
    if (!stream || !payload || !recv) { free(stream); free(payload); free(recv); return OR_CAPACITY; }
    int rc = OR_OK;
    for (int phase = 0; phase < 2 && rc == OR_OK; ++phase) {
        for (int s = 0; s + 1 < R && rc == OR_OK; ++s) {
            for (int q = 0; q < R && rc == OR_OK; ++q) {
                int p = mod(q - 1, R);
                int j = phase == 0 ? mod(q - 2 - s, R) : mod(q - 1 - s, R);
                size_t lo = (size_t)j * L, hi = lo + L;
                if (lo > n) lo = n;
                if (hi > n) hi = n;
                for (size_t c0 = lo; c0 < hi; c0 += chunk) {
                    size_t len = hi - c0 < chunk ? hi - c0 : chunk;
                    const uint16_t *src = (phase == 0 && s == 0) ? x[p] : out[p];
                    memcpy(payload, src + c0, len * 2);
                    size_t sz = or_compress(payload, len, stream, cap);
                    if (sz == 0) { rc = OR_CAPACITY; break; }
                    wire += sz;
                    if (or_decompress(stream, sz, recv, len) != OR_OK) { rc = OR_CORRUPT; break; }
                    for (size_t i = 0; i < len; ++i)
                        out[q][c0 + i] = phase == 0 ? or_hop_bf16(recv[i], x[q][c0 + i]) : recv[i];
                }
            }
        }
    }
    free(stream); free(payload); free(recv);
    if (wire_bytes) *wire_bytes = wire;
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Contention rate                                                           */
/* ------------------------------------------------------------------------ */
/*
 * HOCCL ("HOCCL: Offloading Collective Communication from GPU Cores to
 * Accelerate Distributed Training", section 2, contention rate): the share of
 * compute units held by a traffic class while compute kernels are active.
 * Read as I = integral over t of C(t) * CU(t) / N_CU, divided by the integral
 * of C(t); C(t) = 1 inside any compute interval, CU(t) = the sum of cus[k]
 * over communication intervals k that contain t.  Evaluated exactly on the
 * elementary segments between all interval end points.  Returns -1 when no
 * compute time exists.
 */
static int cmp_double(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return x < y ? -1 : x > y ? 1 : 0;
}

double or_contention_rate(const double *comp_t0, const double *comp_t1, size_t nc,
                          const double *comm_t0, const double *comm_t1, const double *cus,
                          size_t nm, double n_cu)
{
    size_t np = 2 * (nc + nm);
    double *pts = (double *)malloc(sizeof(double) * (np ? np : 1));
    if (!pts) return -1.0;
    size_t k = 0;
    for (size_t i = 0; i < nc; ++i) { pts[k++] = comp_t0[i]; pts[k++] = comp_t1[i]; }
    for (size_t i = 0; i < nm; ++i) { pts[k++] = comm_t0[i]; pts[k++] = comm_t1[i]; }
    qsort(pts, np, sizeof(double), cmp_double);
    double num = 0.0, den = 0.0;
    for (size_t s = 0; s + 1 < np; ++s) {
        double a = pts[s], b = pts[s + 1];
        if (!(b > a)) continue;
        double mid = 0.5 * (a + b);
        int busy = 0;
        for (size_t i = 0; i < nc; ++i) if (comp_t0[i] <= mid && mid < comp_t1[i]) busy = 1;
        if (!busy) continue;
        double cu = 0.0;
        for (size_t i = 0; i < nm; ++i) if (comm_t0[i] <= mid && mid < comm_t1[i]) cu += cus[i];
        den += b - a;
        num += (b - a) * cu / n_cu;
    }
    free(pts);
    return den > 0.0 ? num / den : -1.0;
}

/* ------------------------------------------------------------------------ */
/* Element-wise forms of the scalar rules, for tests over many inputs        */
/* ------------------------------------------------------------------------ */

void or_f32_to_bf16_array(const uint32_t *in, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i) out[i] = or_f32_to_bf16(in[i]);
}

void or_hop_bf16_array(const uint16_t *a, const uint16_t *b, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i) out[i] = or_hop_bf16(a[i], b[i]);
}

void or_hop_f32_array(const uint32_t *a, const uint32_t *b, uint32_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i) out[i] = or_hop_f32(a[i], b[i]);
}
