// launch.hpp -- internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hc.h"

namespace hc {

// One contiguous piece of a ring step for one receiver: dst = hop(a, b) for
// a reduce step (a = what arrived from the sender, b = the receiver's own
// data), dst = a for a copy step.  len in elements.
struct Seg {
  const void* a;
  const void* b;
  void* dst;
  uint64_t len;
  void* dst2 = nullptr;   // a second destination of the same values (reduce-and-send step), or NULL
};

constexpr int kMaxSegs = 64;
constexpr int kWgPerCuBudget = 8;   // workgroups per CU of a CU-budget grid

hipError_t launch_reduce_step(const Seg* segs, int nseg, hc_dtype_t dtype, int cu_budget,
                              hipStream_t stream);
hipError_t launch_copy_step(const Seg* segs, int nseg, size_t elem_bytes, int cu_budget,
                            hipStream_t stream);
// A reduce step that stores each sum twice, at dst and dst2: the last
// reduce-scatter step writing the slice's final sum into its owner's output
// and sending it on into the next rank's output (that rank's first
// all-gather copy).
hipError_t launch_reduce_send_step(const Seg* segs, int nseg, hc_dtype_t dtype, int cu_budget, hipStream_t stream);
// The last reduce-scatter step fused with an SGD update: g = hop(a, b) (or
// g = a when b is NULL, a one-rank "sum"), then dst = dst - lr*g in place
// (dst holds the owner's weights); when the segments carry dst2 (and b), the
// new weights are also sent on into dst2.
hipError_t launch_sgd_step(const Seg* segs, int nseg, hc_dtype_t dtype, float lr, int cu_budget,
                           hipStream_t stream);
// A reduce-scatter step of the bf16 ring with fp32 partials: dst = a + b in
// fp32, b bf16; a is an fp32 partial when a_f32 (else bf16 data); the sum is
// stored as an fp32 partial when dst_f32, else rounded once to bf16 (and,
// when a segment carries dst2, also sent on into dst2).
hipError_t launch_carry_step(const Seg* segs, int nseg, bool a_f32, bool dst_f32, int cu_budget,
                             hipStream_t stream);

// Codec.
hipError_t launch_fill_u32(void* dst, uint32_t value, size_t words, hipStream_t stream);
hipError_t launch_compress(const uint16_t* in, size_t n, void* out, uint64_t* out_bytes,
                           void* ws, hipStream_t stream);
hipError_t launch_decompress(const void* in, size_t in_bytes, uint16_t* out, size_t n,
                             int32_t* status, hipStream_t stream);
size_t compress_ws_bytes(size_t n);
// Stream helpers shared by the codec formats (magic: the format's).
hipError_t launch_empty_stream(void* out, uint32_t magic, uint64_t* out_bytes, hipStream_t stream);
hipError_t launch_check_empty_stream(const void* in, size_t in_bytes, uint32_t magic, int32_t* status,
                                     hipStream_t stream);
// Zeroes the n-element output when *status reports a corrupt stream.
hipError_t launch_zero_if_corrupt(const int32_t* status, uint16_t* out, size_t n, hipStream_t stream);
// Entropy-coded variant (HCE1): per-block canonical Huffman codes for the
// exponent; same workspace as the fixed-length encoder.
hipError_t launch_hce_compress(const uint16_t* in, size_t n, void* out, uint64_t* out_bytes, void* ws,
                               hipStream_t stream);
hipError_t launch_hce_decompress(const void* in, size_t in_bytes, uint16_t* out, size_t n, int32_t* status,
                                 hipStream_t stream);
// Three-round baseline (blocks into slots, prefix of the sizes, coalescing
// copy); the same stream as launch_compress.
size_t staged_ws_bytes(size_t n);
hipError_t launch_compress_staged(const uint16_t* in, size_t n, void* out, uint64_t* out_bytes, void* ws,
                                  hipStream_t stream);
// Table-scope variant: code tables shared by groups of `group` full blocks
// (0: one table for the whole stream).
size_t compress_scoped_ws_bytes(size_t n);
hipError_t launch_compress_scoped(const uint16_t* in, size_t n, void* out, uint64_t* out_bytes, void* ws,
                                  size_t group, hipStream_t stream);

// Compressed ring allreduce (bf16).
size_t compressed_ar_ws_bytes(size_t count, int R);
// events: optional step events (n of them, >= 2R when R > 1, else >= 2).
hipError_t launch_compressed_allreduce(void* const* send, void* const* recv, size_t count, int R,
                                       size_t chunk, void* ws, uint64_t* wire_bytes,
                                       hipEvent_t* events, int n_events, hipStream_t stream);

}  // namespace hc
