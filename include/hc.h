/*
 * hc.h -- C ABI of the MI355X (gfx950) emulated ring AllReduce data path and
 * the lossless bf16 exponent codecs, HCZ1 (fixed-length codes) and HCE1
 * (Huffman codes) (library: libhc.so).
 *
 * The ring is emulated on ONE GPU: R "ranks" are R device buffers in the same
 * HBM; a hop's link transfer is the receiver reading the sender's buffer.  All
 * calls are asynchronous and stream ordered, like the NCCL-style
 * allreduce(sendbuf, recvbuf, count, dtype, op, comm, stream) interface that
 * "CCCL: In-GPU Compression-Coupled Collective Communication" keeps (section
 * 3, "CCCL Overview"); argument errors are found on the host before anything
 * is enqueued.  The only reduction is sum.
 *
 * Memory and ownership
 *   - Every data pointer below is a DEVICE pointer unless it says HOST.
 *     sendbufs/recvbufs are HOST arrays of nranks DEVICE pointers.
 *   - The caller owns every buffer, workspace and stream.  The library never
 *     allocates or frees device memory and keeps no state between calls
 *     except a thread-local copy of the last error message, and the static
 *     device array (about 1 MiB per GPU) of hc_compress_bf16_noalloc.
 *   - Alignment (else HC_ERR_INVALID_ARGUMENT): rank buffers of the
 *     uncompressed ring calls to their element size (16-byte alignment of
 *     every slice takes the vector path, anything else a per-element path);
 *     every pointer of the codec and compressed calls to 16 bytes.
 *   - Buffers of different ranks must not overlap, except for the in-place
 *     forms stated per call.  Sizes are in elements unless named *_bytes.
 *
 * Errors
 *   - HC_ERR_INVALID_ARGUMENT: NULL pointer, nranks outside 1..HC_MAX_RANKS,
 *     misaligned pointer, count constraints, unknown dtype or option value.
 *   - HC_ERR_INSUFFICIENT_CAPACITY: workspace or output capacity too small.
 *   - HC_ERR_UNSUPPORTED: an option the call cannot honour (the copy engine
 *     for hc_compressed_allreduce, or in a process whose HIP runtime would not
 *     put the copies on the DMA engines).
 *   - HC_ERR_DEVICE: a HIP call failed; hc_last_error() has the text.
 *   - HC_ERR_CORRUPT_STREAM: only ever written by the device into the
 *     caller's status word of hc_decompress_bf16 / hc_decompress_bf16_entropy.
 *   The first three are found on the host before anything is enqueued.  An
 *   HC_ERR_DEVICE return can follow launches of the same call that were
 *   already enqueued; the stream then holds a partial operation.  No call
 *   aborts or throws across the ABI.
 */
#ifndef HC_H
#define HC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HC_MAX_RANKS 64
#define HC_BLOCK_ELEMS 16384u        /* codec block: 16384 bf16 = 32 KB */
#define HC_HCZ1_MAGIC 0x315A4348u    /* "HCZ1" little-endian */

/* Every enum of this header also names the ends of the int32 range (the
 * *_RANGE_MIN_ / *_RANGE_MAX_ entries, never valid arguments), so that any
 * 32-bit value a C caller passes is a value of the type in C++ as well: the
 * library's checks then reject unknown values instead of reading a value the
 * type cannot hold. */
typedef enum {
    HC_SUCCESS = 0,
    HC_ERR_INVALID_ARGUMENT = 1,
    HC_ERR_UNSUPPORTED = 2,
    HC_ERR_INSUFFICIENT_CAPACITY = 3,
    HC_ERR_CORRUPT_STREAM = 4,
    HC_ERR_DEVICE = 5,
    HC_STATUS_RANGE_MIN_ = INT32_MIN,
    HC_STATUS_RANGE_MAX_ = INT32_MAX
} hc_status_t;

typedef enum {
    HC_F32 = 0,
    HC_BF16 = 1,
    HC_DTYPE_RANGE_MIN_ = INT32_MIN,
    HC_DTYPE_RANGE_MAX_ = INT32_MAX
} hc_dtype_t;

/* Options.  Pass NULL for the defaults (all fields zero mean default).
 *   chunk_fraction: chunk size as a fraction of the per-rank buffer, default
 *     0.01 ("a chunk is about 1% of the data", "ResCCL: Resource-Efficient
 *     Scheduling for Collective Communication", section 1).  The chunk is
 *     rounded up to 1024 elements (uncompressed) or to whole 16384-element
 *     codec blocks (compressed).  It changes scheduling only, never a value.
 *   cu_budget: 0 = size grids for the whole GPU; k > 0 = launch a persistent
 *     grid sized for k compute units (pair it with a stream from
 *     hc_stream_create_cu_budget(k)).
 *   Environment, read at every call (none is required):
 *     HC_CHUNK_FRACTION (a number in (0, 1]) and HC_CU_BUDGET (an integer in
 *       0..4096) replace the two defaults above where opts is NULL or leaves
 *       the field 0; a malformed value makes every call that takes options
 *       return HC_ERR_INVALID_ARGUMENT, naming the variable.  (The compressed
 *       allreduce, which takes no CU budget, ignores HC_CU_BUDGET.)
 *     HC_LOG (anything but empty or "0") prints each call's plan and each
 *       ring-step launch's shape and tile policy to stderr, one line each,
 *       prefixed "hc: ".
 *     HC_STREAM_STORE_MIN_BYTES (a whole number; default 335544320, 320 MiB):
 *       a ring-step launch that writes at least this many bytes on all CUs
 *       moves one 16-byte vector per lane with non-temporal stores, since its
 *       output no longer fits MI355X's 256 MB Infinity Cache for the next
 *       step to read back; smaller launches use two vectors and ordinary
 *       stores, CU-budget launches four.  Values are the same either way.
 *     HC_CHAIN_MAX_BYTES (a whole number; default 268435456, 256 MiB): an
 *       hc_allreduce whose R buffers hold at most this many bytes runs as
 *       one launch in which each workgroup carries one tile through every
 *       hop in ring order (unless step_events or copy_engine ask for per-step
 *       launches); larger ones launch once per ring step.  When set, it is
 *       also hc_compressed_allreduce's threshold (bytes of its R buffers),
 *       which otherwise always runs as one launch.  Values and wire bytes are
 *       the same either way.
 *     HC_LOOKBACK_SPIN_LIMIT (1..2^32-1; default 2^22): polls a compress
 *       block's look-back makes before the call gives up (see
 *       hc_compress_bf16).
 *   step_events / n_step_events: optional timing hook.  When step_events is
 *     not NULL it holds n_step_events caller-created HIP events (created
 *     with timing enabled), used as step_event_mode says, with steps =
 *     hc_step_count(op, nranks).  Too few events is HC_ERR_INVALID_ARGUMENT.
 *     NULL records nothing; so does a call with nothing to do (count 0).
 *   step_event_mode: 0 = boundaries: step_events[k] is recorded on the stream
 *     right before ring step k and step_events[steps] after the last step
 *     (steps + 1 events), so an interval also holds the gap between two
 *     launches.  1 = kernel stamps (2 * steps events): step k's first kernel
 *     stamps step_events[2k] with its start time and its kernels stamp
 *     step_events[2k+1] with their end time (hipExtLaunchKernel), so an
 *     interval is the step's kernel execution as a kernel trace reports it.
 *     A step that runs no kernel (copy-engine copies; the all-gather step
 *     that the last reduce-scatter step already did) records both events on
 *     the stream around what it enqueues.  Other values are
 *     HC_ERR_INVALID_ARGUMENT.
 *   copy_engine: 0 = all-gather copy steps run as copy kernels on the
 *     compute units; 1 = they run on the GPU's DMA copy engines
 *     (hipMemcpyAsync of kind hipMemcpyDeviceToDeviceNoCU, stream ordered,
 *     one copy per receiver and step), holding no compute unit at all.  This
 *     is the offload of "HOCCL: Offloading Collective Communication from GPU
 *     Cores to Accelerate Distributed Training" (section 2): a copy can leave
 *     the cores, a reduction cannot, so reduce-scatter steps always run on
 *     the compute units.  Applies to hc_all_gather, to the all-gather half of
 *     hc_allreduce and to one-rank copies; hc_compressed_allreduce decodes
 *     during its all-gather and rejects it (HC_ERR_UNSUPPORTED).  Other
 *     values are HC_ERR_INVALID_ARGUMENT.  Which engine serves such a copy
 *     is the HIP runtime's choice: measured on MI355X, the ROCm 7.2 runtime
 *     in /opt/rocm uses the DMA engines (about 60 GB/s per copy, one copy at
 *     a time per stream), while the 7.0 runtime bundled with the PyTorch
 *     2.10 wheel runs the same calls as blit kernels on the compute units.
 *     So a call with copy_engine = 1 in a process whose HIP runtime is older
 *     than 7.2 returns HC_ERR_UNSUPPORTED (nothing is enqueued) instead of
 *     silently using the compute units; hc_copy_engine_available() tells in
 *     advance. */
typedef struct {
    double chunk_fraction;
    int32_t cu_budget;
    int32_t n_step_events;
    hipEvent_t *step_events;
    int32_t copy_engine;
    int32_t step_event_mode;
} hc_opts_t;

/*
 * hc_allreduce -- ring AllReduce (sum) over nranks emulated ranks.
 * "Breaking the computation and communication abstraction barrier in
 * distributed machine learning workloads" ("The idea"): AllReduce is a
 * ReduceScatter followed by an AllGather, and every rank ends with the same
 * full result (local -> replicated).  Runs R-1 recvReduceCopy steps then R-1
 * copy steps ("ResCCL ...", section 1).  At reduce-scatter step s receiver q
 * folds slice (q-2-s) mod R received from q-1 into its own data; at
 * all-gather step s it copies slice (q-1-s) mod R from q-1.  Element i of
 * slice j is therefore hop(...hop(x[j+1][i], x[j+2][i])..., x[j][i]).
 *   fp32: hop = one IEEE binary32 add (round to nearest even, subnormals
 *         kept); bf16: both operands widened exactly to fp32, one add, the
 *         sum rounded to bf16 nearest-even.  A NaN sum becomes the canonical
 *         quiet NaN (0x7FC00000 / 0x7FC0).
 *   sendbufs[r], recvbufs[r]: count elements each.  In place is allowed:
 *   sendbufs[r] == recvbufs[r] for every r.  Slices are ceil(count/R) long
 *   (the last ones short or empty when R does not divide count).
 *   Schedule: up to HC_CHAIN_MAX_BYTES of buffers (256 MiB by default) the
 *   hops run in one launch, each workgroup taking one tile of one slice
 *   through all 2(R-1) hops in order ("ResCCL ...", section 3: dependencies
 *   exist only within a chunk); above it, or with step_events or
 *   copy_engine, one launch per ring step.  Both make the same reads and
 *   writes and give the same bits.
 */
hc_status_t hc_allreduce(void *const *sendbufs, void *const *recvbufs, size_t count,
                         hc_dtype_t dtype, int nranks, const hc_opts_t *opts,
                         hipStream_t stream);

/*
 * hc_allreduce_bf16_f32carry -- the bf16 ring AllReduce of hc_allreduce with
 * the other reading of "fp32 accumulation, bf16 round-to-nearest-even
 * output": the reduce-scatter carries fp32 partials and the sum is rounded to
 * bf16 once, by the slice's owner at the last reduce-scatter step.  Same ring,
 * slices, chunks and fold order as hc_allreduce: element i of slice j is
 * bf16(((f(x[j+1][i]) + f(x[j+2][i])) + ...) + f(x[j][i])) with f the exact
 * widening and every + one fp32 add (a NaN sum becomes the canonical NaN);
 * the all-gather copies the bf16 result.  With 2 ranks this equals
 * hc_allreduce; with 1 it is a copy.  Partials cost 4 bytes instead of 2, so
 * a middle reduce-scatter hop moves 10 bytes per element instead of 6.
 *   sendbufs[r], recvbufs[r]: count bf16 elements each; in place is allowed
 *   (sendbufs[r] == recvbufs[r] for every r).
 *   d_ws: >= hc_workspace_bytes(HC_OP_ALLREDUCE_F32_CARRY, count, nranks,
 *   HC_BF16) bytes, 16-byte aligned, overlapping no rank buffer: two fp32
 *   partial slots per rank (ping-pong between steps).  May be NULL when
 *   nranks <= 2 (no partial is stored).  The caller owns it; its contents
 *   after the call are unspecified.
 *   Errors as hc_allreduce, plus HC_ERR_INSUFFICIENT_CAPACITY for a short
 *   workspace; nothing is enqueued on an argument error.
 */
hc_status_t hc_allreduce_bf16_f32carry(void *const *sendbufs, void *const *recvbufs, size_t count,
                                       int nranks, void *d_ws, size_t ws_bytes, const hc_opts_t *opts,
                                       hipStream_t stream);

/*
 * hc_reduce_scatter -- ring ReduceScatter (sum): rank r receives slice r of
 * the elementwise sum ("Breaking the computation and communication
 * abstraction barrier ...", "The idea": each rank keeps its 1/N slice;
 * local -> sliced).  Same hop and fold order as hc_allreduce.
 *   sendbufs[r]: recvcount*nranks elements; recvbufs[r]: recvcount elements.
 *   In place is allowed: recvbufs[r] == sendbufs[r] + r*recvcount elements.
 *   d_ws: device workspace of at least hc_workspace_bytes(HC_OP_REDUCE_SCATTER,
 *   recvcount*nranks, nranks, dtype) bytes; it holds the partials in flight.
 */
hc_status_t hc_reduce_scatter(void *const *sendbufs, void *const *recvbufs, size_t recvcount,
                              hc_dtype_t dtype, int nranks, void *d_ws, size_t ws_bytes,
                              const hc_opts_t *opts, hipStream_t stream);

/*
 * hc_all_gather -- ring AllGather: every rank receives the concatenation of
 * all ranks' sendbufs, slice j = rank j's data (sliced -> replicated, same
 * page).  Step 0 also copies each rank's own data into its own output.
 *   sendbufs[r]: sendcount elements; recvbufs[r]: sendcount*nranks elements.
 *   In place is allowed: sendbufs[r] == recvbufs[r] + r*sendcount elements.
 */
hc_status_t hc_all_gather(void *const *sendbufs, void *const *recvbufs, size_t sendcount,
                          hc_dtype_t dtype, int nranks, const hc_opts_t *opts,
                          hipStream_t stream);

/*
 * hc_allreduce_sgd -- the allreduce of gradients fused with an SGD update of
 * the weights: "Breaking the computation and communication abstraction
 * barrier in distributed machine learning workloads" ("The idea") moves an
 * elementwise optimizer update between the ReduceScatter and the AllGather,
 * so that each rank updates only the slice whose sum it holds and the
 * AllGather spreads updated weights instead of summed gradients.
 *   grads[r], weights[r]: count elements each, dtype HC_F32 or HC_BF16,
 *     element-aligned; all 2*nranks buffers pairwise disjoint.
 *   g = the ring allreduce sum of the grads, exactly as hc_allreduce computes
 *     it (same fold order, same per-hop rounding).  For slice j (the
 *     hc_allreduce slicing) the new weight is weights[j] - lr*g, the product
 *     and the difference rounded once each in fp32 (bf16: operands widened
 *     exactly, result rounded to nearest even; a NaN result is the canonical
 *     quiet NaN).  On return every weights[r] holds the new weights; slice j
 *     comes from rank j's weights before the call (when every rank holds the
 *     same weights, as in data-parallel training, that is simply w - lr*g).
 *   grads are the reduction's scratch: their contents after the call are
 *     partial sums, unspecified.
 *   lr: any finite float (not finite: HC_ERR_INVALID_ARGUMENT).
 *   opts: chunk_fraction, cu_budget, step_events (2*(nranks-1) steps, 1 for
 *     one rank) and copy_engine (the all-gather copies) as for hc_allreduce.
 * Asynchronous on stream; argument errors are detected before anything is
 * enqueued.
 */
hc_status_t hc_allreduce_sgd(void *const *grads, void *const *weights, size_t count, hc_dtype_t dtype,
                             int nranks, float lr, const hc_opts_t *opts, hipStream_t stream);

/* Largest HCZ1 stream for n bf16 elements (every block stored raw):
 * 32 + round_up(8*n_blocks, 16) + sum over blocks of 16 + round_up(2*m, 16). */
size_t hc_compress_bound_bf16(size_t n);

/*
 * hc_compress_bf16 -- lossless bf16 compression into one HCZ1 stream.
 * "CCCL ...", section 4.1: sign and fraction are sent raw, the 8-bit exponent
 * is coded from a frequency table; section 4.3: each block builds its own
 * table and uses fixed-length codes; section 4.4: one pass, each block writes
 * straight into the output; section 5 "Handling data alignment": a partial
 * tail block is stored raw.
 * Format (little-endian, all padding zero): 32-byte header {u32 magic
 * 0x315A4348, u32 block_elems 16384, u64 n, u32 n_blocks, u32 flags 0, u64
 * total_bytes}; u64 rec_off[n_blocks] padded to 16 bytes; the records in
 * block order.  Record: 16-byte header {u8 mode (0 raw, 1 coded), u8 b, u16
 * 0, u32 m, u32 n_esc, u32 rec_bytes}; raw: m words padded to 16; coded
 * (m == 16384 only): dictionary of the K = 2^b-1 most frequent exponents
 * (count descending, exponent ascending) in max(16, 2^b) bytes; b code
 * planes of 2048 bytes (bit i%8 of byte i/8 of plane k = bit k of code[i],
 * code = dictionary index or K for an escape); the sign/fraction plane
 * sm[i] = sign<<7 | fraction (16384 bytes); the escaped exponents in index
 * order, padded to 16.  b is the smallest 1..7 with the fewest bytes; a block
 * is raw when that is not below 16 + 32768 bytes.
 *   d_in: n bf16 words.  d_out: out_cap >= hc_compress_bound_bf16(n) bytes.
 *   d_out_bytes: one device u64, receives the stream size; it receives 0
 *   (and the stream is not valid) only if a block's wait for its
 *   predecessors' sizes ran past its bound (about four million polls).
 *   d_ws: >= hc_workspace_bytes(HC_OP_COMPRESS, n, 1, HC_BF16) bytes (block
 *   offsets in flight).  Calls sharing a workspace must not overlap.
 */
hc_status_t hc_compress_bf16(const uint16_t *d_in, size_t n, void *d_out, size_t out_cap,
                             uint64_t *d_out_bytes, void *d_ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * hc_compress_bf16_noalloc -- hc_compress_bf16 without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The same
 * kernels, the same stream byte for byte.  The look-back workspace is a
 * static device array inside the library (8320 + 8 * 131072 bytes, about
 * 1 MiB), one copy per GPU, held until the process ends; its address is
 * taken once per device on that device's first call.  The call allocates
 * nothing (no hipMalloc, no allocating library routine) and clears the part
 * of the array it uses with a fill kernel on the stream.
 *   n: at most 131072 * 16384 = 2^31 elements, else
 *   HC_ERR_INSUFFICIENT_CAPACITY (nothing is enqueued).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (on different streams, or from several threads) race and may write
 *   wrong streams; order them on one stream.
 *   Other arguments and errors as hc_compress_bf16.
 */
hc_status_t hc_compress_bf16_noalloc(const uint16_t *d_in, size_t n, void *d_out, size_t out_cap,
                                     uint64_t *d_out_bytes, hipStream_t stream);

/*
 * hc_compress_bf16_scoped -- hc_compress_bf16 with code tables shared by
 * groups of blocks.  "CCCL ...", section 4.3 weighs one global table (more
 * work before any block can be coded) against a table per block (the
 * overhead of many small tables) and picks the per-block one; this call
 * makes the choice a parameter so both ends can be measured.
 *   table_blocks: G >= 1 groups the full blocks in order, G at a time (the
 *   last group may be shorter); 0 puts every full block in one group.  A
 *   group's dictionary is its summed exponent histogram ranked count
 *   descending, exponent ascending; its b (1..7) is the one with the fewest
 *   summed coded bytes over its blocks, ties to the smaller b.  Each full
 *   block is coded with its group's dictionary and b unless that record
 *   would not be below 16 + 32768 bytes, then it is raw; the partial tail
 *   block is raw.  Each record still carries its dictionary, so the result
 *   is an ordinary HCZ1 stream for hc_decompress_bf16, and G = 1 writes the
 *   same bytes as hc_compress_bf16.
 *   d_ws: >= hc_workspace_bytes(HC_OP_COMPRESS_SCOPED, n, 1, HC_BF16) bytes
 *   (independent of G).  Other arguments and errors as hc_compress_bf16.
 */
hc_status_t hc_compress_bf16_scoped(const uint16_t *d_in, size_t n, void *d_out, size_t out_cap,
                                    uint64_t *d_out_bytes, size_t table_blocks, void *d_ws,
                                    size_t ws_bytes, hipStream_t stream);

/*
 * hc_compress_bf16_staged -- hc_compress_bf16 in three global rounds, the
 * design "CCCL ...", section 4.4 replaces: every block encodes into a
 * fixed-size temporary slot (16 + 32768 bytes), a prefix over the record
 * sizes places the records, and a coalescing copy writes them into the
 * stream.  The same encoder and format: the stream equals hc_compress_bf16's
 * byte for byte.  For measuring the single-round design against it.
 *   d_ws: >= hc_workspace_bytes(HC_OP_COMPRESS_STAGED, n, 1, HC_BF16) bytes
 *   (the slots, about 2.0 bytes per element).  Other arguments and errors as
 *   hc_compress_bf16.
 */
hc_status_t hc_compress_bf16_staged(const uint16_t *d_in, size_t n, void *d_out, size_t out_cap,
                                    uint64_t *d_out_bytes, void *d_ws, size_t ws_bytes,
                                    hipStream_t stream);

/*
 * hc_compress_bf16_entropy -- lossless bf16 compression with an entropy-coded
 * exponent: one "HCE1" stream.  "CCCL ...", section 4.1 codes the exponent
 * from a frequency table with sign and fraction raw, and section 6.5
 * compares the fixed-length core with an entropy coder whose output is
 * smaller by under 7%; here each full block codes its exponents with its own
 * canonical Huffman code (lengths limited to 12 bits; codes assigned as in
 * RFC 1951, section 3.2.2), the same container and single-pass writer as
 * hc_compress_bf16.
 * Format (little-endian, all padding zero): the HCZ1 container with magic
 * 0x31454348.  Record: 16-byte header {u8 mode (0 raw, 2 coded), u8 lmax (12
 * coded, 0 raw), u16 n_sym (exponents present; 0 raw), u32 m, u32 n_words
 * (0 raw), u32 rec_bytes}; raw: m words padded to 16; coded (m == 16384
 * only): code length of exponent e (0 absent, 1..12) in the low nibble of
 * byte 16 + e/2 for even e, the high nibble for odd e; bytes 144..16527 the
 * sign/fraction plane sm[i] = sign<<7 | fraction; from byte 16528 the
 * n_words 32-bit words, padded to 16: rec_bytes = 16528 +
 * round_up(4*n_words, 16).  A full block is coded when that is below
 * 16 + 32768 bytes, else raw; the partial tail block is raw.
 * Code construction: leaves in increasing count, equal counts by decreasing
 * exponent; the lighter of (next leaf, next merged node) is taken first, a
 * leaf on a tie; a single exponent gets length 1.  Lengths over 12 become 12,
 * then while the Kraft sum exceeds 1 the longest code shorter than 12
 * (ties: smallest count, then largest exponent) grows by one bit.
 * Word layout: 64 lanes, lane j takes elements 64*i + j (step i = 0..255);
 * its codes, most significant bit first, form a bit stream whose bit b is bit
 * b%32 of its word b/32.  Word w of a lane is stored at the first step whose
 * code ends past bit 32*w of that stream, and the words are stored in (that
 * step, lane) order -- the order in which a decoder running the 64 lanes in
 * lockstep needs them.
 *   d_ws: >= hc_workspace_bytes(HC_OP_COMPRESS_ENTROPY, n, 1, HC_BF16)
 *   bytes.  Other arguments and errors as hc_compress_bf16 (the bound is
 *   hc_compress_bound_bf16(n)).
 */
hc_status_t hc_compress_bf16_entropy(const uint16_t *d_in, size_t n, void *d_out, size_t out_cap,
                                     uint64_t *d_out_bytes, void *d_ws, size_t ws_bytes,
                                     hipStream_t stream);

/*
 * hc_decompress_bf16_entropy -- exact inverse of hc_compress_bf16_entropy.
 * Arguments and errors as hc_decompress_bf16; besides the container, a coded
 * record is rejected when its lengths exceed 12 or break the Kraft
 * inequality, n_sym disagrees with them, a code is missing, the words do not
 * run out exactly at the last code, or a padding bit is set.
 */
hc_status_t hc_decompress_bf16_entropy(const void *d_in, size_t in_bytes, uint16_t *d_out, size_t n,
                                       int32_t *d_status, hipStream_t stream);

/*
 * hc_decompress_bf16 -- exact inverse of hc_compress_bf16.
 *   d_in: in_bytes readable bytes holding a stream of n elements (the stream
 *   may be shorter than in_bytes).  d_out: n bf16 words.  d_status: one
 *   device int32, required; set to HC_SUCCESS, or to HC_ERR_CORRUPT_STREAM
 *   when any field fails validation (magic, block size, n, block count,
 *   contiguous in-bounds offsets, record sizes against the format, b in
 *   1..7, escape count, zero padding) -- then d_out is left all zero.  Reads
 *   never go past in_bytes, whatever the stream holds.
 */
hc_status_t hc_decompress_bf16(const void *d_in, size_t in_bytes, uint16_t *d_out, size_t n,
                               int32_t *d_status, hipStream_t stream);

/*
 * hc_compressed_allreduce -- the ring of hc_allreduce on bf16 with every hop
 * payload sent compressed ("CCCL ...", section 5, "Selective compression":
 * the sender compresses what it sends, the receiver decompresses what it
 * receives and reduces it with its own uncompressed data).  Reduce-scatter
 * hop: decompress -> bf16 hop -> compress (the last one also writes the
 * output); all-gather hop: decompress into the output and forward the same
 * bytes.  Chunks are whole codec blocks; a slice's unaligned end travels as a
 * raw block.  Lossless, so the result is bit-identical to hc_allreduce.
 *   sendbufs/recvbufs: as hc_allreduce (bf16 only; in place allowed).
 *   d_ws: >= hc_workspace_bytes(HC_OP_COMPRESSED_ALLREDUCE, count, nranks,
 *   HC_BF16) bytes: two wire buffers per rank, one fixed-size slot per codec
 *   block (the preallocated regions of "CCCL ...", section 4.4).
 *   d_wire_bytes: optional device u64; receives the bytes that would cross
 *   the links: the sum over every (hop, chunk) stream of its HCZ1 size.
 *   Schedule: one launch, one workgroup per codec block and slice, each
 *   carrying its block through every hop in ring order, with the wire slots
 *   indexed by slice; with step_events, or beyond HC_CHAIN_MAX_BYTES when that
 *   is set, one launch per ring step.  Same records, wire bytes and output
 *   either way.
 */
hc_status_t hc_compressed_allreduce(void *const *sendbufs, void *const *recvbufs, size_t count,
                                    int nranks, void *d_ws, size_t ws_bytes,
                                    uint64_t *d_wire_bytes, const hc_opts_t *opts,
                                    hipStream_t stream);

typedef enum {
    HC_OP_REDUCE_SCATTER = 0,
    HC_OP_COMPRESS = 1,
    HC_OP_COMPRESSED_ALLREDUCE = 2,
    HC_OP_ALLREDUCE = 3,
    HC_OP_ALL_GATHER = 4,
    HC_OP_COMPRESS_SCOPED = 5,
    HC_OP_COMPRESS_ENTROPY = 6,
    HC_OP_COMPRESS_STAGED = 7,
    HC_OP_ALLREDUCE_F32_CARRY = 8,
    HC_OP_RANGE_MIN_ = INT32_MIN,
    HC_OP_RANGE_MAX_ = INT32_MAX
} hc_op_t;

/* Workspace bytes for an operation; count = elements per rank buffer
 * (the send buffer for reduce-scatter, the input for compress).  Returns 0
 * on invalid arguments and for operations that need no workspace. */
size_t hc_workspace_bytes(hc_op_t op, size_t count, int nranks, hc_dtype_t dtype);

/* Ring steps of an operation (for hc_opts_t.step_events): allreduce 2(R-1),
 * reduce-scatter R-1, all-gather R-1 (step 0 includes the local copies),
 * compressed allreduce 2R-1 (the first compression is step 0); an operation
 * over one rank counts 1.  Returns -1 for an unknown op or nranks. */
int hc_step_count(hc_op_t op, int nranks);

/*
 * hc_stream_create_cu_budget -- a HIP stream whose kernels may run only on k
 * compute units (hipExtStreamCreateWithCUMask, default priority), for
 * running a collective beside compute on fewer CUs; "HOCCL: Offloading
 * Collective Communication from GPU Cores to Accelerate Distributed Training"
 * (section 2) measures the share of cores such traffic holds while compute
 * runs.  The k CUs are spread evenly over the GPU's XCDs and shader engines
 * (measured with hc_cu_census: k = 8, 16, 32, 64 give exactly k CUs, k/8 on
 * every XCD).  *out receives the stream; the caller destroys it with
 * hc_stream_destroy.  Same as hc_stream_create_cu_range(0, k, out).
 */
hc_status_t hc_stream_create_cu_budget(int k, hipStream_t *out);

/* A stream limited to CU mask bits [first, first + k) (0 <= first, k >= 1,
 * first + k <= the CU count; else HC_ERR_INVALID_ARGUMENT).  Bits are handed
 * out round-robin over the XCDs, so a run is an even spread and
 * hc_stream_create_cu_range(k, ncu - k) holds exactly the CUs that
 * hc_stream_create_cu_budget(k) leaves free: compute on the one beside
 * communication on the other shares no CU. */
hc_status_t hc_stream_create_cu_range(int first, int k, hipStream_t *out);
hc_status_t hc_stream_destroy(hipStream_t stream);

/*
 * hc_cu_census -- where the workgroups of a launch on `stream` run: the
 * evidence that a CU-budget stream holds exactly the compute units it was
 * given ("HOCCL ...", section 2: the share of cores that communication holds
 * while compute runs is the quantity measured).  Launches n_workgroups
 * one-wave workgroups; each holds its CU for hold_us microseconds (a bounded
 * wait, so that the launch spreads over every CU the stream may use), then
 * writes d_ids[2w] = its HW_ID register (bits 8..15 hold the CU, shader
 * array and shader engine numbers) and d_ids[2w + 1] = its XCC_ID register
 * (bits 0..3: the XCD).  A CU is identified by (XCC_ID & 15, HW_ID bits
 * 8..15).
 *   d_ids: 2 * n_workgroups device u32, 4-byte aligned.  n_workgroups:
 *   1..65536; hold_us: 0..100000.  Asynchronous on stream.
 */
hc_status_t hc_cu_census(uint32_t *d_ids, int n_workgroups, int hold_us, hipStream_t stream);

/* Chunk size in elements for a per-rank buffer of count elements
 * (align = 1024 uncompressed, 16384 compressed); 0 on invalid input. */
size_t hc_chunk_elems(size_t count, double chunk_fraction, size_t align);

/* One Transfer(srcRank, dstRank, step, chunkId, opType) task of the ring
 * ("ResCCL ...", section 3), with the element range it moves. */
typedef struct {
    int32_t src, dst, step, chunk;
    int32_t op;        /* 1 = recvReduceCopy (reduce-scatter), 2 = copy (all-gather) */
    int32_t slice;
    uint64_t off, len; /* element range inside the per-rank buffer */
} hc_task_t;

/* Host-only: the allreduce task list the launcher executes (reduce-scatter
 * steps then all-gather steps; receiver-major, then chunk, in each step).
 * Returns the number of tasks; writes at most cap (tasks may be NULL). */
size_t hc_ring_tasks(int nranks, size_t count, size_t chunk, hc_task_t *tasks, size_t cap);

/* 1 when this process's HIP runtime runs copy_engine copies on the DMA
 * engines (runtime 7.2 or later), else 0: then copy_engine = 1 is
 * HC_ERR_UNSUPPORTED. */
int hc_copy_engine_available(void);

const char *hc_status_string(hc_status_t status);
const char *hc_last_error(void);  /* thread-local, "" when none */
const char *hc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HC_H */
