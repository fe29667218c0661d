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

// The caller's step events (hc_opts_t.step_events) of one call.  Mode 0
// records one event on the stream at every step boundary.  Mode 1 gives each
// step two events that its kernels stamp themselves: the step's first kernel
// stamps ev[2k] with its start time and every kernel of the step stamps
// ev[2k+1] with its end time, so that an interval is the kernels' own
// execution, as a kernel trace measures it, without the gaps between
// launches.  A step that launches no kernel records both events on the
// stream around whatever it enqueues (copy-engine copies, or nothing).
struct Tap {
  hipEvent_t* ev = nullptr;
  int n = 0, k = 0, mode = 0, steps = 0;
  bool open = false;
  hipStream_t stream = nullptr;   // of the first mark
  // At the start of every step and once after the last: mode 0 records the
  // next boundary event; mode 1 closes the open step and opens the next.
  hipError_t mark(hipStream_t s);
  // Records every event not recorded yet (steps that had no work, at the
  // end); the destructor calls it too, so that every event of a call that
  // marked a step ends up recorded.
  hipError_t finish(hipStream_t s);
  ~Tap();
};

// Launches a ring-step kernel (all of them go through here): a plain
// hipLaunchKernel, or, while a mode-1 step is open on this thread,
// hipExtLaunchKernel with the step's start and end events.
hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, hipStream_t stream);
// Tells an open mode-1 step that work other than a kernel (copy-engine
// copies) follows: its start event is recorded on the stream now and its
// end event when the step closes.
hipError_t stamp_host_work(hipStream_t stream);
constexpr int kWgPerCuBudget = 8;   // workgroups per CU of a CU-budget grid

// HC_LOG set to anything but "" or "0": every call prints its plan, and every
// ring-step launch its shape, to stderr, one line each, prefixed "hc: ".
bool log_enabled();
void log_line(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

hipError_t launch_reduce_step(const Seg* segs, int nseg, hc_dtype_t dtype, int cu_budget,
                              hipStream_t stream);
hipError_t launch_copy_step(const Seg* segs, int nseg, size_t elem_bytes, int cu_budget,
                            hipStream_t stream);
// The whole ring allreduce in one launch, one tile per workgroup carried
// through every hop in ring order (see chain_kernel).  send/recv: host
// arrays of R device pointers.
hipError_t launch_chain_allreduce(void* const* send, void* const* recv, size_t count, size_t es, int R,
                                  int cu_budget, hipStream_t stream);
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

// Census of where a launch's workgroups run (see hc_cu_census).
hipError_t launch_cu_census(uint32_t* ids, uint32_t n_workgroups, uint32_t hold_us, hipStream_t stream);

// Codec.
// Polls of an unpublished look-back descriptor before a stream encoder's
// walk gives up: HC_LOOKBACK_SPIN_LIMIT from the environment (read at every
// call; an unsigned decimal >= 1), else 2^22.  A small value makes walks give
// up, which the encoders report as a zero-byte stream; tests use it to
// exercise that path.
uint32_t lookback_spin_limit();
hipError_t launch_fill_u32(void* dst, uint32_t value, size_t words, hipStream_t stream);
hipError_t launch_compress(const uint16_t* in, size_t n, void* out, uint64_t* out_bytes,
                           void* ws, hipStream_t stream);
hipError_t launch_decompress(const void* in, size_t in_bytes, uint16_t* out, size_t n,
                             int32_t* status, hipStream_t stream);
size_t compress_ws_bytes(size_t n);
// The allocation-free compress entry point's static scratch: room for the
// look-back workspace of up to kNoAllocMaxBlocks blocks (2^31 elements).
constexpr size_t kNoAllocMaxBlocks = (size_t)1 << 17;
constexpr size_t kNoAllocScratchBytes = 8320 + 8 * kNoAllocMaxBlocks;
constexpr int kMaxDevices = 64;
// This device's address of the static scratch (taken with
// hipGetSymbolAddress on the device's first call, then kept).
hipError_t noalloc_scratch(void** out);
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
// tap: the call's step events (marked once per step and after the last).
hipError_t launch_compressed_allreduce(void* const* send, void* const* recv, size_t count, int R,
                                       size_t chunk, void* ws, uint64_t* wire_bytes, bool one_launch, Tap& tap,
                                       hipStream_t stream);

}  // namespace hc
