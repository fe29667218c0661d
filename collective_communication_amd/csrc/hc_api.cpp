// hc_api.cpp -- the C ABI of libhc: argument checks, the ring launcher, the
// codec and compressed-ring entry points, CU-budget streams.
//
// Every check runs on the host before anything is enqueued; a call that
// returns an error has launched nothing.  Calls are asynchronous on the
// caller's stream and never synchronize it.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <cmath>
#include <vector>

#include "hc.h"
#include "launch.hpp"
#include "schedule.hpp"

#include <hip/hip_ext.h>

extern "C" int hc_step_count(hc_op_t op, int nranks);

namespace hc {

namespace {

// The open mode-1 step of this thread: its two events, and whether a kernel
// (or host work) has stamped its start and a kernel its end.
struct Stamp {
  hipEvent_t start = nullptr, stop = nullptr;
  bool started = false, stopped = false, host = false;
};
thread_local Stamp t_stamp;

hipError_t close_stamp(hipStream_t stream) {
  const Stamp s = t_stamp;
  t_stamp = Stamp{};
  hipError_t e = hipSuccess;
  if (!s.started) e = hipEventRecord(s.start, stream);
  if (e == hipSuccess && (!s.stopped || s.host)) e = hipEventRecord(s.stop, stream);
  return e;
}

}  // namespace

hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, void** args, hipStream_t stream) {
  Stamp& s = t_stamp;
  if (!s.stop) return hipLaunchKernel(fn, grid, block, args, 0, stream);
  hipEvent_t start = s.started ? nullptr : s.start;
  s.started = s.stopped = true;
  return hipExtLaunchKernel(fn, grid, block, args, 0, stream, start, s.stop, 0);
}

hipError_t stamp_host_work(hipStream_t stream) {
  Stamp& s = t_stamp;
  if (!s.stop) return hipSuccess;
  s.host = true;
  if (s.started) return hipSuccess;
  s.started = true;
  return hipEventRecord(s.start, stream);
}

hipError_t Tap::mark(hipStream_t s) {
  if (!ev) return hipSuccess;
  if (!stream) stream = s;
  if (mode == 0) return k < n ? hipEventRecord(ev[k++], s) : hipSuccess;
  hipError_t e = hipSuccess;
  if (open) {
    open = false;
    e = close_stamp(s);
  }
  if (e == hipSuccess && k < steps) {
    t_stamp = Stamp{ev[2 * k], ev[2 * k + 1]};
    open = true;
    ++k;
  }
  return e;
}

hipError_t Tap::finish(hipStream_t s) {
  if (!ev) return hipSuccess;
  hipError_t e = hipSuccess;
  if (mode == 0) {
    while (e == hipSuccess && k <= steps) e = hipEventRecord(ev[k++], s);
    return e;
  }
  if (open) {
    open = false;
    e = close_stamp(s);
  }
  for (; e == hipSuccess && k < steps; ++k) {
    e = hipEventRecord(ev[2 * k], s);
    if (e == hipSuccess) e = hipEventRecord(ev[2 * k + 1], s);
  }
  return e;
}

Tap::~Tap() {
  if (stream) (void)finish(stream);
  if (open) t_stamp = Stamp{};
}

bool log_enabled() {
  const char* e = getenv("HC_LOG");
  return e && *e && strcmp(e, "0") != 0;
}

void log_line(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  fprintf(stderr, "hc: %s\n", buf);
}

}  // namespace hc

namespace {

using hc::Tap;

thread_local std::string g_last_error;

hc_status_t fail(hc_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hc_status_t fail(hc_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hc_status_t device_fail(hipError_t e, const char* where) {
  return fail(HC_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

size_t esize(hc_dtype_t d) { return d == HC_F32 ? 4 : 2; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Whether this process's HIP runtime runs hipMemcpyDeviceToDeviceNoCU copies
// on the DMA engines.  Measured on MI355X: the ROCm 7.2 runtime does; the
// 7.0 runtime bundled with the PyTorch 2.10 wheel runs them as blit kernels
// on the compute units.  Runtimes before 7.2 are therefore treated as not
// offloading (version = major * 10^7 + minor * 10^5 + patch).
bool dma_copies_offload() {
  static const bool ok = [] {
    int v = 0;
    return hipRuntimeGetVersion(&v) == hipSuccess && v >= 70200000;
  }();
  return ok;
}

hc_status_t check_env();
// Measured on MI355X (one allreduce, us, step-per-launch / one launch):
// R=4 x 2^20 fp32 30.6 / 13.7; R=8 x 2^20 bf16 51.7 / 15.8; R=8 x 2^22 bf16
// 75 / 46; R=8 x 2^24 bf16 199 / 149.  Up to the 256 MB Infinity Cache the
// one-launch schedule wins; above it the step-per-launch schedule streams
// every hop through HBM, which is the ring data path this library measures.
constexpr uint64_t kChainMaxBytes = 256ull << 20;
double chunk_fraction(const hc_opts_t* o);
int cu_budget(const hc_opts_t* o);

hc_status_t check_common(int nranks, hc_dtype_t dtype, const hc_opts_t* opts) {
  if (hc_status_t st = check_env()) return st;
  if (nranks < 1 || nranks > HC_MAX_RANKS)
    return fail(HC_ERR_INVALID_ARGUMENT, "nranks %d outside 1..%d", nranks, HC_MAX_RANKS);
  if (dtype != HC_F32 && dtype != HC_BF16)
    return fail(HC_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  if (opts) {
    if (opts->chunk_fraction != 0.0 && !(opts->chunk_fraction > 0.0 && opts->chunk_fraction <= 1.0))
      return fail(HC_ERR_INVALID_ARGUMENT, "chunk_fraction %g outside (0, 1]", opts->chunk_fraction);
    if (opts->cu_budget < 0 || opts->cu_budget > 4096)
      return fail(HC_ERR_INVALID_ARGUMENT, "cu_budget %d outside 0..4096", opts->cu_budget);
    if (opts->n_step_events < 0) return fail(HC_ERR_INVALID_ARGUMENT, "n_step_events < 0");
    if (opts->copy_engine != 0 && opts->copy_engine != 1)
      return fail(HC_ERR_INVALID_ARGUMENT, "copy_engine %d is neither 0 nor 1", opts->copy_engine);
    if (opts->copy_engine == 1 && !dma_copies_offload()) {
      int v = 0;
      (void)hipRuntimeGetVersion(&v);
      return fail(HC_ERR_UNSUPPORTED,
                  "copy_engine: this process's HIP runtime (version %d) runs device-to-device NoCU copies as "
                  "kernels on the compute units, not on the DMA engines", v);
    }
    if (opts->step_event_mode != 0 && opts->step_event_mode != 1)
      return fail(HC_ERR_INVALID_ARGUMENT, "step_event_mode %d is neither 0 nor 1", opts->step_event_mode);
  }
  return HC_SUCCESS;
}

hc_status_t make_tap(const hc_opts_t* o, hc_op_t op, int nranks, Tap* tap) {
  if (!o || !o->step_events) return HC_SUCCESS;
  const int steps = hc_step_count(op, nranks);
  const int need = o->step_event_mode == 1 ? 2 * steps : steps + 1;
  if (o->n_step_events < need)
    return fail(HC_ERR_INVALID_ARGUMENT, "n_step_events %d < %d", o->n_step_events, need);
  tap->ev = o->step_events;
  tap->n = o->n_step_events;
  tap->mode = o->step_event_mode;
  tap->steps = steps;
  return HC_SUCCESS;
}

// Defaults of the chunk fraction and the CU budget, which the environment may
// replace where a call passes no options or leaves the field 0:
// HC_CHUNK_FRACTION (a number in (0, 1]) and HC_CU_BUDGET (an integer in
// 0..4096).  check_common rejects a malformed value before anything runs.
bool env_chunk_fraction(double* out) {
  const char* e = getenv("HC_CHUNK_FRACTION");
  if (!e || !*e) return false;
  char* end = nullptr;
  const double v = strtod(e, &end);
  if (*end != 0 || !(v > 0.0 && v <= 1.0)) return false;
  *out = v;
  return true;
}
bool env_cu_budget(int* out) {
  const char* e = getenv("HC_CU_BUDGET");
  if (!e || !*e) return false;
  char* end = nullptr;
  const long v = strtol(e, &end, 10);
  if (*end != 0 || v < 0 || v > 4096) return false;
  *out = (int)v;
  return true;
}
hc_status_t check_env() {
  const char* f = getenv("HC_CHUNK_FRACTION");
  double fv;
  if (f && *f && !env_chunk_fraction(&fv))
    return fail(HC_ERR_INVALID_ARGUMENT, "environment HC_CHUNK_FRACTION=\"%.64s\" is not a number in (0, 1]", f);
  const char* b = getenv("HC_CU_BUDGET");
  int bv;
  if (b && *b && !env_cu_budget(&bv))
    return fail(HC_ERR_INVALID_ARGUMENT, "environment HC_CU_BUDGET=\"%.64s\" is not an integer in 0..4096", b);
  return HC_SUCCESS;
}

// HC_CHAIN_MAX_BYTES, when set to a whole number: the largest allreduce (bytes
// of its R buffers) that runs as one launch, for both allreduces.
bool env_chain_max_bytes(uint64_t* v) {
  const char* e = getenv("HC_CHAIN_MAX_BYTES");
  if (!e || !*e) return false;
  char* end = nullptr;
  const unsigned long long x = strtoull(e, &end, 10);
  if (*end != 0) return false;
  *v = x;
  return true;
}

// Allreduces whose R buffers hold at most this many bytes run as one launch
// that carries each chunk through every hop (launch_chain_allreduce); larger
// ones launch once per ring step.
uint64_t chain_max_bytes() {
  uint64_t v;
  return env_chain_max_bytes(&v) ? v : kChainMaxBytes;
}

// The compressed allreduce runs as one launch (each codec block of each slice
// through every hop) unless HC_CHAIN_MAX_BYTES is set, which then applies the
// plain allreduce's byte threshold.  Measured on MI355X (us, step-per-launch /
// one launch): R=2 x 2^18 24.4 / 21.6, x 2^25 106 / 101; R=4 x 2^22 70.9 /
// 54.3, x 2^25 257 / 217; R=8 x 2^22 149 / 105, x 2^25 545 / 446.  Every hop
// of a block depends only on the hop before it, so one launch needs no wait
// between workgroups and saves the ramps and tails of 2R-1 launches.
bool compressed_one_launch(size_t count, int nranks) {
  uint64_t v;
  if (env_chain_max_bytes(&v)) return (uint64_t)count * 2u * (uint64_t)nranks <= v;
  return true;
}

double chunk_fraction(const hc_opts_t* o) {
  if (o && o->chunk_fraction != 0.0) return o->chunk_fraction;
  double v;
  return env_chunk_fraction(&v) ? v : 0.01;
}
int cu_budget(const hc_opts_t* o) {
  if (o && o->cu_budget != 0) return o->cu_budget;
  int v;
  return env_cu_budget(&v) ? v : 0;
}
bool copy_engine(const hc_opts_t* o) { return o && o->copy_engine == 1; }

// One HC_LOG line for a ring call: its shape and the options in force.
void log_ring(const char* op, int nranks, size_t count, hc_dtype_t dtype, size_t chunk, const hc_opts_t* opts,
              const char* note) {
  if (!hc::log_enabled()) return;
  hc::log_line("%s: ranks=%d count=%zu dtype=%s chunk=%zu cu_budget=%d copy_engine=%d steps=%d%s%s", op, nranks,
               count, dtype == HC_F32 ? "f32" : "bf16", chunk, cu_budget(opts), copy_engine(opts) ? 1 : 0,
               opts && opts->step_events ? (opts->step_event_mode == 1 ? 2 : 1) : 0, note ? " " : "",
               note ? note : "");
}

// One copy step: the segments as one copy kernel on the compute units, or as
// one DMA copy per segment on the copy engines (stream ordered).
hipError_t copy_step(const hc::Seg* segs, int nseg, size_t es, int budget, bool dma, hipStream_t stream) {
  if (!dma) return hc::launch_copy_step(segs, nseg, es, budget, stream);
  if (hipError_t e = hc::stamp_host_work(stream); e != hipSuccess) return e;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].len == 0) continue;
    hipError_t e = hipMemcpyAsync(segs[i].dst, segs[i].a, segs[i].len * es, hipMemcpyDeviceToDeviceNoCU, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Checks a pointer array: non-NULL and aligned to `align` bytes.
hc_status_t check_ptrs(void* const* bufs, int R, const char* name, size_t align) {
  if (!bufs) return fail(HC_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  for (int r = 0; r < R; ++r) {
    if (!bufs[r]) return fail(HC_ERR_INVALID_ARGUMENT, "%s[%d] is NULL", name, r);
    if ((uintptr_t)bufs[r] % align)
      return fail(HC_ERR_INVALID_ARGUMENT, "%s[%d] is not %zu-byte aligned", name, r, align);
  }
  return HC_SUCCESS;
}

// Output ranges must be pairwise disjoint and disjoint from every input range
// except the allowed in-place alias (input r == the given offset inside
// output r, checked by the caller as `inplace_ok`).
hc_status_t check_disjoint(const std::vector<Range>& in, const std::vector<Range>& out,
                           const std::vector<bool>& inplace_ok) {
  for (size_t i = 0; i < out.size(); ++i)
    for (size_t j = i + 1; j < out.size(); ++j)
      if (overlap(out[i], out[j]))
        return fail(HC_ERR_INVALID_ARGUMENT, "recvbufs[%zu] and recvbufs[%zu] overlap", i, j);
  for (size_t i = 0; i < out.size(); ++i)
    for (size_t j = 0; j < in.size(); ++j) {
      if (i == j && inplace_ok[i]) continue;
      if (overlap(out[i], in[j]))
        return fail(HC_ERR_INVALID_ARGUMENT, "recvbufs[%zu] overlaps sendbufs[%zu]", i, j);
    }
  return HC_SUCCESS;
}

const char* cp(const void* p, size_t bytes) { return static_cast<const char*>(p) + bytes; }
char* mp(void* p, size_t bytes) { return static_cast<char*>(p) + bytes; }

// Runs the allreduce task list one ring step per launch: all receivers of a
// step in one kernel, their chunks merged into one segment per receiver.
// The last reduce-scatter step is a reduce-and-send: the receiver that forms
// a slice's final sum writes it into its own output and sends it on into the
// next rank's output, which is that rank's first all-gather copy; that copy
// step then has nothing left to do (its step event is still recorded).  With
// the copy engine the first all-gather copy stays a copy of its own.
hc_status_t run_allreduce(void* const* send, void* const* recv, size_t count, hc_dtype_t dtype,
                          int R, size_t chunk, int budget, bool dma, Tap& tap, hipStream_t stream) {
  const size_t es = esize(dtype);
  const bool fuse = !dma;
  std::vector<hc_task_t> tasks = hc::ring_tasks(R, count, chunk);
  size_t k = 0;
  while (k < tasks.size()) {
    const int op = tasks[k].op, step = tasks[k].step;
    const bool send_on = fuse && op == 1 && step == R - 2;
    hc::Seg segs[hc::kMaxSegs];
    int nseg = 0, last_dst = -1;
    uint64_t last_end = 0;
    hipError_t e = tap.mark(stream);
    if (e != hipSuccess) return device_fail(e, "hipEventRecord");
    if (fuse && op != 1 && step == 0) {   // done by the reduce-and-send step
      while (k < tasks.size() && tasks[k].op == op && tasks[k].step == step) ++k;
      continue;
    }
    auto launch = [&]() {
      if (op != 1) return copy_step(segs, nseg, es, budget, dma, stream);
      return send_on ? hc::launch_reduce_send_step(segs, nseg, dtype, budget, stream)
                     : hc::launch_reduce_step(segs, nseg, dtype, budget, stream);
    };
    while (k < tasks.size() && tasks[k].op == op && tasks[k].step == step) {
      const hc_task_t& t = tasks[k];
      const size_t off = t.off * es;
      if (t.dst == last_dst && t.off == last_end) {
        segs[nseg - 1].len += t.len;  // next chunk of the same receiver's slice
      } else {
        if (nseg == hc::kMaxSegs) {   // a full launch (the task order gives one segment per receiver)
          if ((e = launch()) != hipSuccess) return device_fail(e, op == 1 ? "reduce step launch" : "copy step launch");
          nseg = 0;
        }
        segs[nseg].a = (op == 1 && step == 0) ? cp(send[t.src], off) : cp(recv[t.src], off);
        segs[nseg].b = cp(send[t.dst], off);
        segs[nseg].dst = mp(recv[t.dst], off);
        segs[nseg].dst2 = send_on ? mp(recv[(t.dst + 1) % R], off) : nullptr;
        segs[nseg].len = t.len;
        ++nseg;
      }
      last_dst = t.dst;
      last_end = t.off + t.len;
      ++k;
    }
    e = launch();
    if (e != hipSuccess) return device_fail(e, op == 1 ? "reduce step launch" : "copy step launch");
  }
  hipError_t e = tap.mark(stream);
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "hipEventRecord");
}

// The allreduce task list with the reduce-scatter run in place on the
// gradients and its last step fused with the update of the owner's weights;
// the all-gather then spreads the updated weight slices.
hc_status_t run_allreduce_sgd(void* const* grads, void* const* weights, size_t count, hc_dtype_t dtype, int R,
                              size_t chunk, float lr, int budget, bool dma, Tap& tap, hipStream_t stream) {
  const size_t es = esize(dtype);
  const bool fuse = !dma;   // the update step also sends each new slice on (as in run_allreduce)
  std::vector<hc_task_t> tasks = hc::ring_tasks(R, count, chunk);
  size_t k = 0;
  while (k < tasks.size()) {
    const int op = tasks[k].op, step = tasks[k].step;
    const bool last_rs = op == 1 && step == R - 2;
    hc::Seg segs[hc::kMaxSegs];
    int nseg = 0, last_dst = -1;
    uint64_t last_end = 0;
    hipError_t e = tap.mark(stream);
    if (e != hipSuccess) return device_fail(e, "hipEventRecord");
    if (fuse && op != 1 && step == 0) {   // done by the update-and-send step
      while (k < tasks.size() && tasks[k].op == op && tasks[k].step == step) ++k;
      continue;
    }
    auto launch = [&]() {
      if (op != 1) return copy_step(segs, nseg, es, budget, dma, stream);
      return last_rs ? hc::launch_sgd_step(segs, nseg, dtype, lr, budget, stream)
                     : hc::launch_reduce_step(segs, nseg, dtype, budget, stream);
    };
    while (k < tasks.size() && tasks[k].op == op && tasks[k].step == step) {
      const hc_task_t& t = tasks[k];
      const size_t off = t.off * es;
      if (t.dst == last_dst && t.off == last_end) {
        segs[nseg - 1].len += t.len;
      } else {
        if (nseg == hc::kMaxSegs) {   // a full launch (the task order gives one segment per receiver)
          if ((e = launch()) != hipSuccess) return device_fail(e, op == 1 ? "reduce step launch" : "copy step launch");
          nseg = 0;
        }
        if (op == 1) {  // partials stay in the gradients; the last step writes weights
          segs[nseg].a = cp(grads[t.src], off);
          segs[nseg].b = cp(grads[t.dst], off);
          segs[nseg].dst = last_rs ? mp(weights[t.dst], off) : mp(grads[t.dst], off);
          segs[nseg].dst2 = (last_rs && fuse) ? mp(weights[(t.dst + 1) % R], off) : nullptr;
        } else {
          segs[nseg].a = cp(weights[t.src], off);
          segs[nseg].b = nullptr;
          segs[nseg].dst = mp(weights[t.dst], off);
        }
        segs[nseg].len = t.len;
        ++nseg;
      }
      last_dst = t.dst;
      last_end = t.off + t.len;
      ++k;
    }
    e = launch();
    if (e != hipSuccess) return device_fail(e, op == 1 ? "reduce step launch" : "copy step launch");
  }
  hipError_t e = tap.mark(stream);
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "hipEventRecord");
}

// Workspace of the fp32-carry allreduce: two fp32 partial slots per rank of
// Lp = ceil(count/R) rounded up to 64 elements, so that every slot starts
// 256-byte aligned.  No partial is stored with one or two ranks.
size_t carry_slot_elems(size_t count, int R) { return (hc::ceil_div(count, (size_t)R) + 63) & ~(size_t)63; }
size_t carry_ws_bytes(size_t count, int R) {
  return R <= 2 ? 0 : (size_t)R * 2 * carry_slot_elems(count, R) * 4;
}

// The bf16 allreduce with fp32 partials.  Reduce-scatter partials of rank q
// ping-pong between its fp32 workspace slots (q, s%2), each element at its
// offset inside its slice; step 0 reads both operands from the inputs, the
// last step rounds into recvbufs (for two ranks step 0 is the last and this
// is the per-hop bf16 ring).  The all-gather is the usual bf16 copy ring.
hc_status_t run_allreduce_carry(void* const* send, void* const* recv, size_t count, int R, size_t chunk, void* ws,
                                int budget, bool dma, Tap& tap, hipStream_t stream) {
  const size_t es = 2, L = hc::ceil_div(count, (size_t)R), Lp = carry_slot_elems(count, R);
  const bool fuse = !dma;   // the rounding step also sends each slice on (as in run_allreduce)
  std::vector<hc_task_t> tasks = hc::ring_tasks(R, count, chunk);
  size_t k = 0;
  while (k < tasks.size()) {
    const int op = tasks[k].op, step = tasks[k].step;
    const bool first = op == 1 && step == 0, last = op == 1 && step == R - 2;
    hc::Seg segs[hc::kMaxSegs];
    int nseg = 0, last_dst = -1;
    uint64_t last_end = 0;
    hipError_t e = tap.mark(stream);
    if (e != hipSuccess) return device_fail(e, "hipEventRecord");
    if (fuse && op != 1 && step == 0) {   // done by the rounding-and-send step
      while (k < tasks.size() && tasks[k].op == op && tasks[k].step == step) ++k;
      continue;
    }
    auto launch = [&]() {
      return op == 1 ? hc::launch_carry_step(segs, nseg, !first, !last, budget, stream)
                     : copy_step(segs, nseg, es, budget, dma, stream);
    };
    while (k < tasks.size() && tasks[k].op == op && tasks[k].step == step) {
      const hc_task_t& t = tasks[k];
      const size_t off = t.off * es;
      if (t.dst == last_dst && t.off == last_end) {
        segs[nseg - 1].len += t.len;  // next chunk of the same receiver's slice
      } else {
        if (nseg == hc::kMaxSegs) {   // a full launch (the task order gives one segment per receiver)
          if ((e = launch()) != hipSuccess) return device_fail(e, op == 1 ? "reduce step launch" : "copy step launch");
          nseg = 0;
        }
        if (op == 1) {
          const size_t in_slice = t.off - (size_t)t.slice * L;
          segs[nseg].a = first ? cp(send[t.src], off)
                               : cp(ws, ((size_t)(2 * t.src + ((step - 1) & 1)) * Lp + in_slice) * 4);
          segs[nseg].b = cp(send[t.dst], off);
          segs[nseg].dst = last ? mp(recv[t.dst], off) : mp(ws, ((size_t)(2 * t.dst + (step & 1)) * Lp + in_slice) * 4);
          segs[nseg].dst2 = (last && fuse) ? mp(recv[(t.dst + 1) % R], off) : nullptr;
        } else {
          segs[nseg].a = cp(recv[t.src], off);
          segs[nseg].b = nullptr;
          segs[nseg].dst = mp(recv[t.dst], off);
        }
        segs[nseg].len = t.len;
        ++nseg;
      }
      last_dst = t.dst;
      last_end = t.off + t.len;
      ++k;
    }
    e = launch();
    if (e != hipSuccess) return device_fail(e, op == 1 ? "reduce step launch" : "copy step launch");
  }
  hipError_t e = tap.mark(stream);
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "hipEventRecord");
}

// One-rank operations: a single step that copies (or nothing in place).
hc_status_t run_single(const void* src, void* dst, size_t count, size_t es, int budget, bool dma, Tap& tap,
                       hipStream_t stream) {
  hipError_t e = tap.mark(stream);
  if (e == hipSuccess && src != dst) {
    hc::Seg seg{src, nullptr, dst, count};
    e = copy_step(&seg, 1, es, budget, dma, stream);
  }
  if (e == hipSuccess) e = tap.mark(stream);
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "copy launch");
}

}  // namespace

extern "C" {

const char* hc_status_string(hc_status_t s) {
  switch (s) {
    case HC_SUCCESS: return "success";
    case HC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case HC_ERR_UNSUPPORTED: return "unsupported";
    case HC_ERR_INSUFFICIENT_CAPACITY: return "insufficient capacity";
    case HC_ERR_CORRUPT_STREAM: return "corrupt stream";
    case HC_ERR_DEVICE: return "device error";
    default: break;
  }
  return "unknown status";
}

const char* hc_last_error(void) { return g_last_error.c_str(); }

int hc_copy_engine_available(void) { return dma_copies_offload() ? 1 : 0; }
const char* hc_version(void) { return "hc 0.1 gfx950"; }

int hc_step_count(hc_op_t op, int nranks) {
  if (nranks < 1 || nranks > HC_MAX_RANKS) return -1;
  if (nranks == 1) return 1;
  switch (op) {
    case HC_OP_ALLREDUCE:
    case HC_OP_ALLREDUCE_F32_CARRY: return 2 * (nranks - 1);
    case HC_OP_REDUCE_SCATTER: return nranks - 1;
    case HC_OP_ALL_GATHER: return nranks - 1;
    case HC_OP_COMPRESSED_ALLREDUCE: return 2 * nranks - 1;
    case HC_OP_COMPRESS:
    case HC_OP_COMPRESS_SCOPED:
    case HC_OP_COMPRESS_ENTROPY:
    case HC_OP_COMPRESS_STAGED: return -1;
    default: break;
  }
  return -1;
}

size_t hc_chunk_elems(size_t count, double fraction, size_t align) {
  return hc::chunk_elems(count, fraction, align);
}

size_t hc_ring_tasks(int nranks, size_t count, size_t chunk, hc_task_t* tasks, size_t cap) {
  std::vector<hc_task_t> t = hc::ring_tasks(nranks, count, chunk);
  if (tasks)
    for (size_t i = 0; i < t.size() && i < cap; ++i) tasks[i] = t[i];
  return t.size();
}

hc_status_t hc_allreduce(void* const* sendbufs, void* const* recvbufs, size_t count,
                         hc_dtype_t dtype, int nranks, const hc_opts_t* opts, hipStream_t stream) {
  g_last_error.clear();
  hc_status_t st = check_common(nranks, dtype, opts);
  if (st) return st;
  if (count == 0) return HC_SUCCESS;
  if ((st = check_ptrs(sendbufs, nranks, "sendbufs", esize(dtype)))) return st;
  if ((st = check_ptrs(recvbufs, nranks, "recvbufs", esize(dtype)))) return st;
  const size_t es = esize(dtype);
  if (count > ((size_t)1 << 40)) return fail(HC_ERR_INVALID_ARGUMENT, "count %zu too large", count);
  std::vector<Range> in, out;
  std::vector<bool> ok;
  for (int r = 0; r < nranks; ++r) {
    in.push_back({(uintptr_t)sendbufs[r], (uintptr_t)sendbufs[r] + count * es});
    out.push_back({(uintptr_t)recvbufs[r], (uintptr_t)recvbufs[r] + count * es});
    ok.push_back(sendbufs[r] == recvbufs[r]);
  }
  if ((st = check_disjoint(in, out, ok))) return st;
  Tap tap;
  if ((st = make_tap(opts, HC_OP_ALLREDUCE, nranks, &tap))) return st;
  const size_t chunk = hc::chunk_elems(count, chunk_fraction(opts), 1024);
  if (nranks == 1) {
    log_ring("allreduce", nranks, count, dtype, chunk, opts, "(one rank: a copy)");
    return run_single(sendbufs[0], recvbufs[0], count, es, cu_budget(opts), copy_engine(opts), tap, stream);
  }
  if (!copy_engine(opts) && !tap.ev && (uint64_t)count * es * (uint64_t)nranks <= chain_max_bytes()) {
    log_ring("allreduce", nranks, count, dtype, chunk, opts, "(one launch: each tile through every hop)");
    hipError_t e = hc::launch_chain_allreduce(sendbufs, recvbufs, count, es, nranks, cu_budget(opts), stream);
    return e == hipSuccess ? HC_SUCCESS : device_fail(e, "chain launch");
  }
  log_ring("allreduce", nranks, count, dtype, chunk, opts, "(one segment per receiver and step: a step's chunks are merged)");
  return run_allreduce(sendbufs, recvbufs, count, dtype, nranks, chunk, cu_budget(opts), copy_engine(opts), tap,
                       stream);
}

hc_status_t hc_allreduce_bf16_f32carry(void* const* sendbufs, void* const* recvbufs, size_t count, int nranks,
                                       void* d_ws, size_t ws_bytes, const hc_opts_t* opts, hipStream_t stream) {
  g_last_error.clear();
  hc_status_t st = check_common(nranks, HC_BF16, opts);
  if (st) return st;
  if (count == 0) return HC_SUCCESS;
  if ((st = check_ptrs(sendbufs, nranks, "sendbufs", 2))) return st;
  if ((st = check_ptrs(recvbufs, nranks, "recvbufs", 2))) return st;
  if (count > ((size_t)1 << 40)) return fail(HC_ERR_INVALID_ARGUMENT, "count %zu too large", count);
  std::vector<Range> in, out;
  std::vector<bool> ok;
  for (int r = 0; r < nranks; ++r) {
    in.push_back({(uintptr_t)sendbufs[r], (uintptr_t)sendbufs[r] + count * 2});
    out.push_back({(uintptr_t)recvbufs[r], (uintptr_t)recvbufs[r] + count * 2});
    ok.push_back(sendbufs[r] == recvbufs[r]);
  }
  if ((st = check_disjoint(in, out, ok))) return st;
  const size_t need = carry_ws_bytes(count, nranks);
  if (need) {
    if (!d_ws) return fail(HC_ERR_INVALID_ARGUMENT, "d_ws is NULL");
    if (!aligned16(d_ws)) return fail(HC_ERR_INVALID_ARGUMENT, "d_ws is not 16-byte aligned");
    if (ws_bytes < need) return fail(HC_ERR_INSUFFICIENT_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
    Range wr{(uintptr_t)d_ws, (uintptr_t)d_ws + need};
    for (int r = 0; r < nranks; ++r)
      if (overlap(wr, in[r]) || overlap(wr, out[r]))
        return fail(HC_ERR_INVALID_ARGUMENT, "d_ws overlaps rank %d buffers", r);
  }
  Tap tap;
  if ((st = make_tap(opts, HC_OP_ALLREDUCE_F32_CARRY, nranks, &tap))) return st;
  log_ring("allreduce_bf16_f32carry", nranks, count, HC_BF16, hc::chunk_elems(count, chunk_fraction(opts), 1024), opts,
           "(one segment per receiver and step)");
  if (nranks == 1)
    return run_single(sendbufs[0], recvbufs[0], count, 2, cu_budget(opts), copy_engine(opts), tap, stream);
  const size_t chunk = hc::chunk_elems(count, chunk_fraction(opts), 1024);
  return run_allreduce_carry(sendbufs, recvbufs, count, nranks, chunk, d_ws, cu_budget(opts), copy_engine(opts),
                             tap, stream);
}

hc_status_t hc_allreduce_sgd(void* const* grads, void* const* weights, size_t count, hc_dtype_t dtype,
                             int nranks, float lr, const hc_opts_t* opts, hipStream_t stream) {
  g_last_error.clear();
  hc_status_t st = check_common(nranks, dtype, opts);
  if (st) return st;
  if (!(lr == lr) || lr == INFINITY || lr == -INFINITY)
    return fail(HC_ERR_INVALID_ARGUMENT, "lr is not finite");
  if (count == 0) return HC_SUCCESS;
  if ((st = check_ptrs(grads, nranks, "grads", esize(dtype)))) return st;
  if ((st = check_ptrs(weights, nranks, "weights", esize(dtype)))) return st;
  if (count > ((size_t)1 << 40)) return fail(HC_ERR_INVALID_ARGUMENT, "count %zu too large", count);
  const size_t es = esize(dtype);
  // Every buffer is written: all 2R ranges must be pairwise disjoint.
  std::vector<Range> all;
  for (int r = 0; r < nranks; ++r) all.push_back({(uintptr_t)grads[r], (uintptr_t)grads[r] + count * es});
  for (int r = 0; r < nranks; ++r) all.push_back({(uintptr_t)weights[r], (uintptr_t)weights[r] + count * es});
  for (size_t i = 0; i < all.size(); ++i)
    for (size_t j = i + 1; j < all.size(); ++j)
      if (overlap(all[i], all[j]))
        return fail(HC_ERR_INVALID_ARGUMENT, "buffers %zu and %zu overlap (grads 0..R-1, then weights)", i, j);
  Tap tap;
  if ((st = make_tap(opts, HC_OP_ALLREDUCE, nranks, &tap))) return st;
  log_ring("allreduce_sgd", nranks, count, dtype, hc::chunk_elems(count, chunk_fraction(opts), 1024), opts,
           "(one segment per receiver and step)");
  if (nranks == 1) {  // the sum is the one gradient: one update step
    hipError_t e = tap.mark(stream);
    hc::Seg seg{grads[0], nullptr, weights[0], count};
    if (e == hipSuccess) e = hc::launch_sgd_step(&seg, 1, dtype, lr, cu_budget(opts), stream);
    if (e == hipSuccess) e = tap.mark(stream);
    return e == hipSuccess ? HC_SUCCESS : device_fail(e, "update launch");
  }
  const size_t chunk = hc::chunk_elems(count, chunk_fraction(opts), 1024);
  return run_allreduce_sgd(grads, weights, count, dtype, nranks, chunk, lr, cu_budget(opts), copy_engine(opts),
                           tap, stream);
}

size_t hc_workspace_bytes(hc_op_t op, size_t count, int nranks, hc_dtype_t dtype) {
  if (nranks < 1 || nranks > HC_MAX_RANKS) return 0;
  if (dtype != HC_F32 && dtype != HC_BF16) return 0;
  switch (op) {
    case HC_OP_REDUCE_SCATTER:
      if (count % (size_t)nranks) return 0;
      return 2 * count * esize(dtype);          // two slices per rank, R ranks
    case HC_OP_COMPRESS:
      return hc::compress_ws_bytes(count);
    case HC_OP_COMPRESS_SCOPED:
      return hc::compress_scoped_ws_bytes(count);
    case HC_OP_COMPRESS_ENTROPY:
      return hc::compress_ws_bytes(count);
    case HC_OP_COMPRESS_STAGED:
      return hc::staged_ws_bytes(count);
    case HC_OP_COMPRESSED_ALLREDUCE:
      if (dtype != HC_BF16) return 0;
      return hc::compressed_ar_ws_bytes(count, nranks);
    case HC_OP_ALLREDUCE_F32_CARRY:
      if (dtype != HC_BF16) return 0;
      return carry_ws_bytes(count, nranks);
    case HC_OP_ALLREDUCE:
    case HC_OP_ALL_GATHER:
      return 0;
    default: break;
  }
  return 0;
}

hc_status_t hc_reduce_scatter(void* const* sendbufs, void* const* recvbufs, size_t recvcount,
                              hc_dtype_t dtype, int nranks, void* d_ws, size_t ws_bytes,
                              const hc_opts_t* opts, hipStream_t stream) {
  g_last_error.clear();
  hc_status_t st = check_common(nranks, dtype, opts);
  if (st) return st;
  if (recvcount == 0) return HC_SUCCESS;
  if ((st = check_ptrs(sendbufs, nranks, "sendbufs", esize(dtype)))) return st;
  if ((st = check_ptrs(recvbufs, nranks, "recvbufs", esize(dtype)))) return st;
  if (recvcount > ((size_t)1 << 40))
    return fail(HC_ERR_INVALID_ARGUMENT, "recvcount %zu too large", recvcount);
  const int R = nranks;
  const size_t es = esize(dtype), L = recvcount, n = L * (size_t)R;
  std::vector<Range> in, out;
  std::vector<bool> ok;
  for (int r = 0; r < R; ++r) {
    in.push_back({(uintptr_t)sendbufs[r], (uintptr_t)sendbufs[r] + n * es});
    out.push_back({(uintptr_t)recvbufs[r], (uintptr_t)recvbufs[r] + L * es});
    ok.push_back(recvbufs[r] == cp(sendbufs[r], (size_t)r * L * es));
  }
  if ((st = check_disjoint(in, out, ok))) return st;
  Tap tap;
  if ((st = make_tap(opts, HC_OP_REDUCE_SCATTER, R, &tap))) return st;
  log_ring("reduce_scatter", R, n, dtype, hc::chunk_elems(n, chunk_fraction(opts), 1024), opts,
           "(one segment per receiver and step)");
  if (R == 1) return run_single(sendbufs[0], recvbufs[0], L, es, cu_budget(opts), copy_engine(opts), tap, stream);
  const size_t need = 2 * n * es;
  if (!d_ws) return fail(HC_ERR_INVALID_ARGUMENT, "d_ws is NULL");
  if (!aligned16(d_ws)) return fail(HC_ERR_INVALID_ARGUMENT, "d_ws is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(HC_ERR_INSUFFICIENT_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
  Range wr{(uintptr_t)d_ws, (uintptr_t)d_ws + need};
  for (int r = 0; r < R; ++r)
    if (overlap(wr, in[r]) || overlap(wr, out[r]))
      return fail(HC_ERR_INVALID_ARGUMENT, "d_ws overlaps rank %d buffers", r);
  // Partials of rank q ping-pong between ws slot (q, s%2); the last step lands
  // in recvbufs[q].  Chunks of one receiver merge into one segment per step.
  const int budget = cu_budget(opts);
  for (int s = 0; s + 1 < R; ++s) {
    hc::Seg segs[hc::kMaxSegs];
    for (int q = 0; q < R; ++q) {
      const int p = hc::ring_mod(q - 1, R);
      const int j = hc::ring_slice(0, q, s, R);
      const void* a = s == 0 ? cp(sendbufs[p], (size_t)j * L * es)
                             : cp(d_ws, ((size_t)(2 * p + ((s - 1) & 1)) * L) * es);
      void* dst = (s == R - 2) ? recvbufs[q] : mp(d_ws, ((size_t)(2 * q + (s & 1)) * L) * es);
      segs[q] = hc::Seg{a, cp(sendbufs[q], (size_t)j * L * es), dst, L};
    }
    hipError_t e = tap.mark(stream);
    if (e == hipSuccess) e = hc::launch_reduce_step(segs, R, dtype, budget, stream);
    if (e != hipSuccess) return device_fail(e, "reduce step launch");
  }
  hipError_t e = tap.mark(stream);
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "hipEventRecord");
}

hc_status_t hc_all_gather(void* const* sendbufs, void* const* recvbufs, size_t sendcount,
                          hc_dtype_t dtype, int nranks, const hc_opts_t* opts, hipStream_t stream) {
  g_last_error.clear();
  hc_status_t st = check_common(nranks, dtype, opts);
  if (st) return st;
  if (sendcount == 0) return HC_SUCCESS;
  if ((st = check_ptrs(sendbufs, nranks, "sendbufs", esize(dtype)))) return st;
  if ((st = check_ptrs(recvbufs, nranks, "recvbufs", esize(dtype)))) return st;
  if (sendcount > ((size_t)1 << 40))
    return fail(HC_ERR_INVALID_ARGUMENT, "sendcount %zu too large", sendcount);
  const int R = nranks;
  const size_t es = esize(dtype), L = sendcount, n = L * (size_t)R;
  std::vector<Range> in, out;
  std::vector<bool> ok;
  for (int r = 0; r < R; ++r) {
    in.push_back({(uintptr_t)sendbufs[r], (uintptr_t)sendbufs[r] + L * es});
    out.push_back({(uintptr_t)recvbufs[r], (uintptr_t)recvbufs[r] + n * es});
    ok.push_back(sendbufs[r] == cp(recvbufs[r], (size_t)r * L * es));
  }
  if ((st = check_disjoint(in, out, ok))) return st;
  const int budget = cu_budget(opts);
  Tap tap;
  if ((st = make_tap(opts, HC_OP_ALL_GATHER, R, &tap))) return st;
  log_ring("all_gather", R, n, dtype, hc::chunk_elems(n, chunk_fraction(opts), 1024), opts,
           "(one segment per receiver and step)");
  hipError_t e0 = tap.mark(stream);
  if (e0 != hipSuccess) return device_fail(e0, "hipEventRecord");
  // Local copies (each rank's own slice into its own output), skipped in place.
  {
    hc::Seg segs[hc::kMaxSegs];
    int nseg = 0;
    for (int r = 0; r < R; ++r)
      if (!ok[r]) segs[nseg++] = hc::Seg{sendbufs[r], nullptr, mp(recvbufs[r], (size_t)r * L * es), L};
    hipError_t e = copy_step(segs, nseg, es, budget, copy_engine(opts), stream);
    if (e != hipSuccess) return device_fail(e, "local copy launch");
  }
  for (int s = 0; s + 1 < R; ++s) {
    hc::Seg segs[hc::kMaxSegs];
    for (int q = 0; q < R; ++q) {
      const int p = hc::ring_mod(q - 1, R);
      const int j = hc::ring_slice(1, q, s, R);
      const void* a = s == 0 ? sendbufs[p] : cp(recvbufs[p], (size_t)j * L * es);
      segs[q] = hc::Seg{a, nullptr, mp(recvbufs[q], (size_t)j * L * es), L};
    }
    hipError_t e = s > 0 ? tap.mark(stream) : hipSuccess;  // step 0 began before the local copies
    if (e == hipSuccess) e = copy_step(segs, R, es, budget, copy_engine(opts), stream);
    if (e != hipSuccess) return device_fail(e, "copy step launch");
  }
  hipError_t e = tap.mark(stream);
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "hipEventRecord");
}

size_t hc_compress_bound_bf16(size_t n) {
  const size_t B = HC_BLOCK_ELEMS, nb = hc::ceil_div(n, B);
  size_t total = 32 + hc::round_up(8 * nb, 16);
  if (nb) total += (nb - 1) * (16 + 2 * B) + 16 + hc::round_up(2 * (n - (nb - 1) * B), 16);
  return total;
}

namespace {

enum class Coder { kPerBlock, kScoped, kEntropy, kStaged };

// The compress entry points: per-block fixed-length tables, tables shared by
// groups of blocks, or per-block Huffman codes (HCE1).
hc_status_t compress_common(const uint16_t* d_in, size_t n, void* d_out, size_t out_cap, uint64_t* d_out_bytes,
                            void* d_ws, size_t ws_bytes, Coder coder, size_t table_blocks, hipStream_t stream) {
  const bool scoped = coder == Coder::kScoped;
  g_last_error.clear();
  if (!d_out || !d_out_bytes || !d_ws || (n && !d_in))
    return fail(HC_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if ((d_in && !aligned16(d_in)) || !aligned16(d_out) || !aligned16(d_ws) || ((uintptr_t)d_out_bytes & 7u))
    return fail(HC_ERR_INVALID_ARGUMENT, "misaligned pointer argument");
  if (n > ((size_t)1 << 40)) return fail(HC_ERR_INVALID_ARGUMENT, "n %zu too large", n);
  const size_t bound = hc_compress_bound_bf16(n);
  if (out_cap < bound)
    return fail(HC_ERR_INSUFFICIENT_CAPACITY, "out_cap %zu < bound %zu", out_cap, bound);
  const size_t need = scoped                     ? hc::compress_scoped_ws_bytes(n)
                      : coder == Coder::kStaged ? hc::staged_ws_bytes(n)
                                                : hc::compress_ws_bytes(n);
  if (ws_bytes < need)
    return fail(HC_ERR_INSUFFICIENT_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
  Range ir{(uintptr_t)d_in, (uintptr_t)d_in + 2 * n}, orr{(uintptr_t)d_out, (uintptr_t)d_out + bound},
      wr{(uintptr_t)d_ws, (uintptr_t)d_ws + need};
  if (overlap(ir, orr) || overlap(ir, wr) || overlap(orr, wr))
    return fail(HC_ERR_INVALID_ARGUMENT, "input, output and workspace must not overlap");
  if (hc::log_enabled()) {
    static const char* const kName[] = {"compress", "compress_scoped", "compress_entropy", "compress_staged"};
    hc::log_line("%s: n=%zu blocks=%zu out_cap=%zu table_blocks=%zu", kName[(int)coder], n,
                 hc::ceil_div(n, (size_t)HC_BLOCK_ELEMS), out_cap, table_blocks);
  }
  hipError_t e = coder == Coder::kScoped
                     ? hc::launch_compress_scoped(d_in, n, d_out, d_out_bytes, d_ws, table_blocks, stream)
                 : coder == Coder::kEntropy ? hc::launch_hce_compress(d_in, n, d_out, d_out_bytes, d_ws, stream)
                 : coder == Coder::kStaged  ? hc::launch_compress_staged(d_in, n, d_out, d_out_bytes, d_ws, stream)
                                            : hc::launch_compress(d_in, n, d_out, d_out_bytes, d_ws, stream);
  if (e == hipErrorNotSupported) return fail(HC_ERR_UNSUPPORTED, "compress not built");
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "compress launch");
}

}  // namespace

hc_status_t hc_compress_bf16(const uint16_t* d_in, size_t n, void* d_out, size_t out_cap,
                             uint64_t* d_out_bytes, void* d_ws, size_t ws_bytes, hipStream_t stream) {
  return compress_common(d_in, n, d_out, out_cap, d_out_bytes, d_ws, ws_bytes, Coder::kPerBlock, 1, stream);
}

hc_status_t hc_compress_bf16_noalloc(const uint16_t* d_in, size_t n, void* d_out, size_t out_cap,
                                     uint64_t* d_out_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (n > hc::kNoAllocMaxBlocks * (size_t)HC_BLOCK_ELEMS)
    return fail(HC_ERR_INSUFFICIENT_CAPACITY, "n %zu exceeds the static scratch's %zu elements", n,
                hc::kNoAllocMaxBlocks * (size_t)HC_BLOCK_ELEMS);
  if (!d_out || !d_out_bytes || (n && !d_in)) return fail(HC_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if ((d_in && !aligned16(d_in)) || !aligned16(d_out) || ((uintptr_t)d_out_bytes & 7u))
    return fail(HC_ERR_INVALID_ARGUMENT, "misaligned pointer argument");
  const size_t bound = hc_compress_bound_bf16(n);
  if (out_cap < bound) return fail(HC_ERR_INSUFFICIENT_CAPACITY, "out_cap %zu < bound %zu", out_cap, bound);
  Range ir{(uintptr_t)d_in, (uintptr_t)d_in + 2 * n}, orr{(uintptr_t)d_out, (uintptr_t)d_out + bound};
  if (n && overlap(ir, orr)) return fail(HC_ERR_INVALID_ARGUMENT, "input and output must not overlap");
  void* ws = nullptr;
  hipError_t e = hc::noalloc_scratch(&ws);
  if (e != hipSuccess) return device_fail(e, "static scratch address");
  if (hc::log_enabled())
    hc::log_line("compress_noalloc: n=%zu blocks=%zu out_cap=%zu (static workspace)", n,
                 hc::ceil_div(n, (size_t)HC_BLOCK_ELEMS), out_cap);
  e = hc::launch_compress(d_in, n, d_out, d_out_bytes, ws, stream);
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "compress launch");
}

hc_status_t hc_compress_bf16_scoped(const uint16_t* d_in, size_t n, void* d_out, size_t out_cap,
                                    uint64_t* d_out_bytes, size_t table_blocks, void* d_ws, size_t ws_bytes,
                                    hipStream_t stream) {
  return compress_common(d_in, n, d_out, out_cap, d_out_bytes, d_ws, ws_bytes, Coder::kScoped, table_blocks,
                         stream);
}

hc_status_t hc_compress_bf16_staged(const uint16_t* d_in, size_t n, void* d_out, size_t out_cap,
                                    uint64_t* d_out_bytes, void* d_ws, size_t ws_bytes, hipStream_t stream) {
  return compress_common(d_in, n, d_out, out_cap, d_out_bytes, d_ws, ws_bytes, Coder::kStaged, 1, stream);
}

hc_status_t hc_compress_bf16_entropy(const uint16_t* d_in, size_t n, void* d_out, size_t out_cap,
                                     uint64_t* d_out_bytes, void* d_ws, size_t ws_bytes, hipStream_t stream) {
  return compress_common(d_in, n, d_out, out_cap, d_out_bytes, d_ws, ws_bytes, Coder::kEntropy, 1, stream);
}

namespace {

hc_status_t decompress_common(const void* d_in, size_t in_bytes, uint16_t* d_out, size_t n, int32_t* d_status,
                              bool entropy, hipStream_t stream) {
  g_last_error.clear();
  if (!d_in || !d_status || (n && !d_out)) return fail(HC_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned16(d_in) || (d_out && !aligned16(d_out)) || ((uintptr_t)d_status & 3u))
    return fail(HC_ERR_INVALID_ARGUMENT, "misaligned pointer argument");
  if (n > ((size_t)1 << 40)) return fail(HC_ERR_INVALID_ARGUMENT, "n %zu too large", n);
  Range ir{(uintptr_t)d_in, (uintptr_t)d_in + in_bytes}, orr{(uintptr_t)d_out, (uintptr_t)d_out + 2 * n};
  if (n && overlap(ir, orr)) return fail(HC_ERR_INVALID_ARGUMENT, "input and output overlap");
  if (hc::log_enabled())
    hc::log_line("%s: n=%zu in_bytes=%zu", entropy ? "decompress_entropy" : "decompress", n, in_bytes);
  hipError_t e = entropy ? hc::launch_hce_decompress(d_in, in_bytes, d_out, n, d_status, stream)
                         : hc::launch_decompress(d_in, in_bytes, d_out, n, d_status, stream);
  if (e == hipErrorNotSupported) return fail(HC_ERR_UNSUPPORTED, "decompress not built");
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "decompress launch");
}

}  // namespace

hc_status_t hc_decompress_bf16(const void* d_in, size_t in_bytes, uint16_t* d_out, size_t n,
                               int32_t* d_status, hipStream_t stream) {
  return decompress_common(d_in, in_bytes, d_out, n, d_status, false, stream);
}

hc_status_t hc_decompress_bf16_entropy(const void* d_in, size_t in_bytes, uint16_t* d_out, size_t n,
                                       int32_t* d_status, hipStream_t stream) {
  return decompress_common(d_in, in_bytes, d_out, n, d_status, true, stream);
}

hc_status_t hc_compressed_allreduce(void* const* sendbufs, void* const* recvbufs, size_t count,
                                    int nranks, void* d_ws, size_t ws_bytes, uint64_t* d_wire_bytes,
                                    const hc_opts_t* opts, hipStream_t stream) {
  g_last_error.clear();
  hc_status_t st = check_common(nranks, HC_BF16, opts);
  if (st) return st;
  if (opts && opts->cu_budget != 0)
    return fail(HC_ERR_UNSUPPORTED, "cu_budget is not supported by the compressed allreduce");
  if (copy_engine(opts))
    return fail(HC_ERR_UNSUPPORTED, "the compressed allreduce decodes during its all-gather: no copy_engine");
  if (d_wire_bytes && ((uintptr_t)d_wire_bytes & 7u))
    return fail(HC_ERR_INVALID_ARGUMENT, "d_wire_bytes is not 8-byte aligned");
  if ((st = check_ptrs(sendbufs, nranks, "sendbufs", 16))) return st;
  if ((st = check_ptrs(recvbufs, nranks, "recvbufs", 16))) return st;
  if (count > ((size_t)1 << 40)) return fail(HC_ERR_INVALID_ARGUMENT, "count %zu too large", count);
  std::vector<Range> in, out;
  std::vector<bool> ok;
  for (int r = 0; r < nranks; ++r) {
    in.push_back({(uintptr_t)sendbufs[r], (uintptr_t)sendbufs[r] + count * 2});
    out.push_back({(uintptr_t)recvbufs[r], (uintptr_t)recvbufs[r] + count * 2});
    ok.push_back(sendbufs[r] == recvbufs[r]);
  }
  if ((st = check_disjoint(in, out, ok))) return st;
  const size_t need = hc::compressed_ar_ws_bytes(count, nranks);
  if (!d_ws) return fail(HC_ERR_INVALID_ARGUMENT, "d_ws is NULL");
  if (!aligned16(d_ws)) return fail(HC_ERR_INVALID_ARGUMENT, "d_ws is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(HC_ERR_INSUFFICIENT_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
  Range wr{(uintptr_t)d_ws, (uintptr_t)d_ws + need};
  for (int r = 0; r < nranks; ++r)
    if (overlap(wr, in[r]) || overlap(wr, out[r]))
      return fail(HC_ERR_INVALID_ARGUMENT, "d_ws overlaps rank %d buffers", r);
  Tap tap;
  if ((st = make_tap(opts, HC_OP_COMPRESSED_ALLREDUCE, nranks, &tap))) return st;
  const size_t chunk = hc::chunk_elems(count, chunk_fraction(opts), HC_BLOCK_ELEMS);
  const bool one_launch = !tap.ev && compressed_one_launch(count, nranks);
  log_ring("compressed_allreduce", nranks, count, HC_BF16, chunk, opts,
           one_launch ? "(one launch: each codec block of each slice through every hop)"
                      : "(chunks are whole codec blocks; each chunk's hop payload is its own stream)");
  hipError_t e = hc::launch_compressed_allreduce(sendbufs, recvbufs, count, nranks, chunk, d_ws, d_wire_bytes,
                                                 one_launch, tap, stream);
  if (e == hipSuccess) e = tap.finish(stream);
  if (e == hipErrorNotSupported) return fail(HC_ERR_UNSUPPORTED, "compressed allreduce not built");
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "compressed allreduce launch");
}

hc_status_t hc_stream_create_cu_range(int first, int k, hipStream_t* out) {
  g_last_error.clear();
  if (!out) return fail(HC_ERR_INVALID_ARGUMENT, "out is NULL");
  if (k < 1) return fail(HC_ERR_INVALID_ARGUMENT, "k %d < 1", k);
  if (first < 0) return fail(HC_ERR_INVALID_ARGUMENT, "first %d < 0", first);
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return device_fail(e, "hipDeviceGetAttribute");
  if (k > ncu || first > ncu - k)
    return fail(HC_ERR_INVALID_ARGUMENT, "CUs [%d, %d) outside 0..%d", first, first + k, ncu);
  // Mask bits [first, first + k): the runtime hands mask bits out round-robin
  // over the XCDs and then the shader engines (bit i: XCD i % 8 on MI355X),
  // so a run of bits is an even spread, and two disjoint runs are two
  // disjoint sets of CUs (hc_cu_census measures both).
  std::vector<uint32_t> mask((size_t)(ncu + 31) / 32, 0u);
  for (int i = first; i < first + k; ++i) mask[(size_t)i / 32] |= 1u << (i % 32);
  e = hipExtStreamCreateWithCUMask(out, (uint32_t)mask.size(), mask.data());
  if (e != hipSuccess) return device_fail(e, "hipExtStreamCreateWithCUMask");
  return HC_SUCCESS;
}

hc_status_t hc_stream_create_cu_budget(int k, hipStream_t* out) { return hc_stream_create_cu_range(0, k, out); }

hc_status_t hc_cu_census(uint32_t* d_ids, int n_workgroups, int hold_us, hipStream_t stream) {
  g_last_error.clear();
  if (!d_ids) return fail(HC_ERR_INVALID_ARGUMENT, "d_ids is NULL");
  if ((uintptr_t)d_ids & 3u) return fail(HC_ERR_INVALID_ARGUMENT, "d_ids is not 4-byte aligned");
  if (n_workgroups < 1 || n_workgroups > 65536)
    return fail(HC_ERR_INVALID_ARGUMENT, "n_workgroups %d outside 1..65536", n_workgroups);
  if (hold_us < 0 || hold_us > 100000) return fail(HC_ERR_INVALID_ARGUMENT, "hold_us %d outside 0..100000", hold_us);
  const hipError_t e = hc::launch_cu_census(d_ids, (uint32_t)n_workgroups, (uint32_t)hold_us, stream);
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "census launch");
}

hc_status_t hc_stream_destroy(hipStream_t stream) {
  g_last_error.clear();
  hipError_t e = hipStreamDestroy(stream);
  return e == hipSuccess ? HC_SUCCESS : device_fail(e, "hipStreamDestroy");
}

}  // extern "C"
