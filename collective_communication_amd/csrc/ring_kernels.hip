// ring_kernels.hip -- the recvReduceCopy hop and the copy hop of an emulated
// ring step, for gfx950.
//
// "ResCCL: Resource-Efficient Scheduling for Collective Communication"
// (section 1) names the primitives: a receiver folds what its predecessor
// sent into its own data (recvReduceCopy) during reduce-scatter, and copies
// it (recv) during all-gather.  "CCCL: In-GPU Compression-Coupled
// Collective Communication" (Figure 2, section 5) shows NCCL's version moving
// 16-byte packs; here every lane moves 16-byte vectors too (4 fp32 or 8
// bf16), one to four of them per operand in flight (the launch policy
// below), so a wave64 issues fully coalesced 1 KB loads, marked
// non-temporal.  Both kernels are HBM bound: a reduce hop reads 2
// and writes 1 element per element of the step, a copy hop reads 1, writes 1.
//
// The last reduce-scatter step of the fused allreduce + SGD update
// ("Breaking the computation and communication abstraction barrier in
// distributed machine learning workloads", "The idea": the optimizer update
// moves between the ReduceScatter and the AllGather) reads the owner's weight
// from the destination and writes the updated weight there: 3 reads, 1 write
// per element.
//
// One launch covers one whole ring step: up to 64 segments (one per
// receiver), cut into 4096-element (bf16) / 2048-element (fp32) tiles, one
// tile per workgroup, or a persistent grid-stride loop when the caller gives
// a CU budget.
#include <cstdlib>

#include "common.hpp"
#include "launch.hpp"

namespace hc {
namespace {

// Tuning knobs (compile-time).  Non-temporal loads are the fastest on every
// hop: the hint matters on the received operand, whose lines would otherwise
// push the partials that the next step reads out of the caches.
#ifndef HC_RING_UNROLL
#define HC_RING_UNROLL 2
#endif
#ifndef HC_RING_NT_LOAD
#define HC_RING_NT_LOAD 1
#endif
#ifndef HC_RING_NT_A
#define HC_RING_NT_A HC_RING_NT_LOAD
#endif
#ifndef HC_RING_NT_B
#define HC_RING_NT_B HC_RING_NT_LOAD
#endif
#ifndef HC_RING_NT_STORE
#define HC_RING_NT_STORE 0
#endif
constexpr int kUnroll = HC_RING_UNROLL;  // 16-byte vectors per operand in flight per lane (carry hops)

// How a step launch moves its tiles, chosen per launch on the host
// (launch_step).  Measured on MI355X with the R=8 bf16 reduce hop:
//  - kPolicyCached: 2 vectors per operand per lane, ordinary stores.  The
//    next hop reads what this one writes; while a launch writes no more than
//    the 256 MB Infinity Cache holds, much of that comes back from the cache
//    (R=8 x 2^26: 6.8 TB/s; non-temporal stores lose that and run 6.2-6.4).
//  - kPolicyStream: 1 vector per operand per lane, non-temporal stores, for
//    launches that write more than the cache holds, so every byte goes to
//    HBM anyway (R=8 x 2^28: 6.4 TB/s against 5.9 with the cached policy).
//  - kPolicyBudget: 4 vectors per operand per lane, ordinary stores, on a CU
//    budget, where each CU's rate is bound by the loads it keeps in flight
//    (R=8 x 2^28 on 8 CUs: 471 GB/s against 451 with 2).
constexpr int kPolicyCached = 0;
constexpr int kPolicyStream = 1;
constexpr int kPolicyBudget = 2;
__host__ __device__ constexpr int policy_unroll(int p) { return p == kPolicyStream ? 1 : p == kPolicyBudget ? 4 : 2; }
__host__ __device__ constexpr bool policy_nt_store(int p) { return p == kPolicyStream; }
// Launches that write at least this many bytes take kPolicyStream (between
// the 256 MiB that still gain from the cache and the 512 MiB that do not);
// HC_STREAM_STORE_MIN_BYTES in the environment replaces it.
constexpr uint64_t kStreamStoreMinBytes = 320ull << 20;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 ld_stream(const char* p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return ld16(p);
  }
}
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ uint2 ld_stream8(const char* p) {
  if constexpr (NT) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
  } else {
    return *reinterpret_cast<const uint2*>(p);
  }
}
template <bool NT>
__device__ __forceinline__ void st_stream(char* p, uint4 v) {
  if constexpr (NT) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
  } else {
    st16(p, v);
  }
}

// Step operations.
constexpr int kCopy = 0;     // dst = a
constexpr int kReduce = 1;   // dst = hop(a, b)
constexpr int kSgd = 2;      // dst = dst - lr * hop(a, b)
constexpr int kSgdOne = 3;   // dst = dst - lr * a (one rank: the sum is a)
constexpr int kReduceSend = 4;   // dst = dst2 = hop(a, b)
constexpr int kSgdSend = 5;      // dst = dst2 = dst - lr * hop(a, b)

struct SegArgs {
  const void* a[kMaxSegs];
  const void* b[kMaxSegs];
  void* dst[kMaxSegs];
  void* dst2[kMaxSegs];          // second destination (kReduceSend only)
  uint64_t len[kMaxSegs];
  uint32_t tile0[kMaxSegs + 1];  // first tile of each segment; tile0[nseg] = total
  int32_t nseg;
  float lr;
};

template <int ES>
__device__ __forceinline__ uint32_t scalar_hop(uint32_t a, uint32_t b) {
  if constexpr (ES == 4) {
    return hop_f32(a, b);
  } else {
    return bf16_rne(f32_bits(bits_f32(a << 16) + bits_f32(b << 16)));
  }
}

template <int ES>
__device__ __forceinline__ uint32_t scalar_sgd(uint32_t w, uint32_t g, float lr) {
  if constexpr (ES == 4) {
    return sgd_f32(w, g, lr);
  } else {
    return bf16_rne(f32_bits(bits_f32(w << 16) - lr * bits_f32(g << 16)));
  }
}

template <int ES>
__device__ __forceinline__ uint4 vec_sgd(uint4 w, uint4 g, float lr) {
  if constexpr (ES == 4) return sgd_f32x4(w, g, lr);
  else return sgd_bf16x8(w, g, lr);
}

template <int ES>
__device__ __forceinline__ uint32_t ld_elem(const char* p, uint64_t i) {
  if constexpr (ES == 4) return reinterpret_cast<const uint32_t*>(p)[i];
  else return reinterpret_cast<const uint16_t*>(p)[i];
}

template <int ES>
__device__ __forceinline__ void st_elem(char* p, uint64_t i, uint32_t v) {
  if constexpr (ES == 4) reinterpret_cast<uint32_t*>(p)[i] = v;
  else reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)v;
}

template <int ES>
__device__ __forceinline__ uint4 vec_hop(uint4 a, uint4 b) {
  if constexpr (ES == 4) return hop_f32x4(a, b);
  else return hop_bf16x8(a, b);
}

// ES: element bytes (4 fp32, 2 bf16).  OP: kCopy, kReduce (recvReduceCopy),
// kSgd, kSgdOne, and the two that also send their result on (kReduceSend,
// kSgdSend).  VEC: every segment pointer is 16-byte aligned, so whole
// tiles move as 16-byte vectors; otherwise (odd slice offsets) each lane
// moves elements.
template <int ES, int OP, bool VEC, int POLICY>
__global__ __launch_bounds__(kThreads) void step_kernel(SegArgs args) {
  constexpr bool kUsesB = OP == kReduce || OP == kSgd || OP == kReduceSend || OP == kSgdSend;
  constexpr bool kUpdates = OP == kSgd || OP == kSgdOne || OP == kSgdSend;
  constexpr bool kSends = OP == kReduceSend || OP == kSgdSend;
  constexpr int V = 16 / ES;
  constexpr int U = policy_unroll(POLICY);
  constexpr bool NTS = policy_nt_store(POLICY);
  constexpr uint64_t kTile = (uint64_t)kThreads * V * U;
  const uint32_t total = args.tile0[args.nseg];
  const int tid = threadIdx.x;
  for (uint32_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int lo = 0, hi = args.nseg - 1;
    while (lo < hi) {  // last segment whose first tile is <= tile
      const int mid = (lo + hi + 1) >> 1;
      if (args.tile0[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    const uint64_t base = (uint64_t)(tile - args.tile0[s]) * kTile;
    const uint64_t len = args.len[s];
    const char* pa = static_cast<const char*>(args.a[s]);
    const char* pb = static_cast<const char*>(args.b[s]);
    char* pd = static_cast<char*>(args.dst[s]);
    char* pd2 = kSends ? static_cast<char*>(args.dst2[s]) : nullptr;
    if (VEC && base + kTile <= len) {
      uint4 va[U], vb[U], vw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t off = (base + (uint64_t)(u * kThreads + tid) * V) * ES;
        va[u] = ld_stream<HC_RING_NT_A>(pa + off);
        if constexpr (kUsesB) vb[u] = ld_stream<HC_RING_NT_B>(pb + off);
        if constexpr (kUpdates) vw[u] = ld16(pd + off);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t off = (base + (uint64_t)(u * kThreads + tid) * V) * ES;
        if constexpr (OP == kCopy) st_stream<NTS>(pd + off, va[u]);
        else if constexpr (OP == kReduce) st_stream<NTS>(pd + off, vec_hop<ES>(va[u], vb[u]));
        else if constexpr (OP == kReduceSend) {
          const uint4 r = vec_hop<ES>(va[u], vb[u]);
          st_stream<NTS>(pd + off, r);
          st_stream<NTS>(pd2 + off, r);
        }
        else if constexpr (OP == kSgd) st_stream<NTS>(pd + off, vec_sgd<ES>(vw[u], vec_hop<ES>(va[u], vb[u]), args.lr));
        else if constexpr (OP == kSgdSend) {
          const uint4 r = vec_sgd<ES>(vw[u], vec_hop<ES>(va[u], vb[u]), args.lr);
          st_stream<NTS>(pd + off, r);
          st_stream<NTS>(pd2 + off, r);
        }
        else st_stream<NTS>(pd + off, vec_sgd<ES>(vw[u], va[u], args.lr));
      }
    } else {
      const uint64_t end = base + kTile < len ? base + kTile : len;
      for (uint64_t i = base + tid; i < end; i += kThreads) {
        const uint32_t x = ld_elem<ES>(pa, i);
        if constexpr (OP == kCopy) st_elem<ES>(pd, i, x);
        else if constexpr (OP == kReduce) st_elem<ES>(pd, i, scalar_hop<ES>(x, ld_elem<ES>(pb, i)));
        else if constexpr (OP == kReduceSend) {
          const uint32_t r = scalar_hop<ES>(x, ld_elem<ES>(pb, i));
          st_elem<ES>(pd, i, r);
          st_elem<ES>(pd2, i, r);
        }
        else if constexpr (OP == kSgd)
          st_elem<ES>(pd, i, scalar_sgd<ES>(ld_elem<ES>(pd, i), scalar_hop<ES>(x, ld_elem<ES>(pb, i)), args.lr));
        else if constexpr (OP == kSgdSend) {
          const uint32_t r = scalar_sgd<ES>(ld_elem<ES>(pd, i), scalar_hop<ES>(x, ld_elem<ES>(pb, i)), args.lr);
          st_elem<ES>(pd, i, r);
          st_elem<ES>(pd2, i, r);
        }
        else st_elem<ES>(pd, i, scalar_sgd<ES>(ld_elem<ES>(pd, i), x, args.lr));
      }
    }
  }
}

// Reduce-scatter hops of the bf16 ring with fp32 partials (one rounding at
// the end).  AF: the arriving operand a is an fp32 partial (else bf16 data);
// DF: the sum stays an fp32 partial (else it is rounded to bf16, nearest
// even).  b, the receiver's own data, is bf16.  Each sum is one fp32 add of
// exactly widened operands; a NaN sum is the canonical fp32 NaN.  A lane
// moves 4 consecutive elements per access, so every wave instruction covers
// one contiguous range: 1 KB of fp32 or 512 bytes of bf16.
template <bool F32>
__device__ __forceinline__ void carry_load4(const char* p, uint64_t e, uint32_t (&w)[4]) {
  if constexpr (F32) {
    const uint4 v = ld_stream<HC_RING_NT_A>(p + 4 * e);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    const uint2 v = ld_stream8<HC_RING_NT_A>(p + 2 * e);
    w[0] = v.x << 16; w[1] = v.x & 0xFFFF0000u; w[2] = v.y << 16; w[3] = v.y & 0xFFFF0000u;
  }
}

template <bool AF, bool DF, bool VEC>
__global__ __launch_bounds__(kThreads) void carry_kernel(SegArgs args) {
  constexpr int kSub = 2 * kUnroll;                           // 4-element accesses per lane per tile
  constexpr uint64_t kTile = (uint64_t)kThreads * 4 * kSub;
  const uint32_t total = args.tile0[args.nseg];
  const int tid = threadIdx.x;
  for (uint32_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int lo = 0, hi = args.nseg - 1;
    while (lo < hi) {  // last segment whose first tile is <= tile
      const int mid = (lo + hi + 1) >> 1;
      if (args.tile0[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int s = lo;
    const uint64_t base = (uint64_t)(tile - args.tile0[s]) * kTile;
    const uint64_t len = args.len[s];
    const char* pa = static_cast<const char*>(args.a[s]);
    const char* pb = static_cast<const char*>(args.b[s]);
    char* pd = static_cast<char*>(args.dst[s]);
    char* pd2 = DF ? nullptr : static_cast<char*>(args.dst2[s]);   // the rounded sum sent on, or NULL
    if (VEC && base + kTile <= len) {
      uint32_t wa[kSub][4];
      uint2 vb[kSub];
#pragma unroll
      for (int q = 0; q < kSub; ++q) {
        const uint64_t e = base + (uint64_t)(q * kThreads + tid) * 4;
        carry_load4<AF>(pa, e, wa[q]);
        vb[q] = ld_stream8<HC_RING_NT_B>(pb + 2 * e);
      }
#pragma unroll
      for (int q = 0; q < kSub; ++q) {
        const uint64_t e = base + (uint64_t)(q * kThreads + tid) * 4;
        const uint32_t s0 = hop_f32(wa[q][0], vb[q].x << 16), s1 = hop_f32(wa[q][1], vb[q].x & 0xFFFF0000u);
        const uint32_t s2 = hop_f32(wa[q][2], vb[q].y << 16), s3 = hop_f32(wa[q][3], vb[q].y & 0xFFFF0000u);
        if constexpr (DF) {
          st_stream<HC_RING_NT_STORE>(pd + 4 * e, make_uint4(s0, s1, s2, s3));
        } else {
          const uint2 r = make_uint2(bf16_rne(s0) | (bf16_rne(s1) << 16), bf16_rne(s2) | (bf16_rne(s3) << 16));
          *reinterpret_cast<uint2*>(pd + 2 * e) = r;
          if (pd2) *reinterpret_cast<uint2*>(pd2 + 2 * e) = r;
        }
      }
    } else {
      const uint64_t end = base + kTile < len ? base + kTile : len;
      for (uint64_t i = base + tid; i < end; i += kThreads) {
        const uint32_t a = AF ? ld_elem<4>(pa, i) : ld_elem<2>(pa, i) << 16;
        const uint32_t sum = hop_f32(a, ld_elem<2>(pb, i) << 16);
        if constexpr (DF) {
          st_elem<4>(pd, i, sum);
        } else {
          st_elem<2>(pd, i, bf16_rne(sum));
          if (pd2) st_elem<2>(pd2, i, bf16_rne(sum));
        }
      }
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Launch of one fp32-carry reduce-scatter step (see carry_kernel).
template <bool AF, bool DF>
hipError_t launch_carry(const Seg* segs, int nseg, int cu_budget, hipStream_t stream) {
  constexpr uint64_t kTile = (uint64_t)kThreads * 8 * kUnroll;   // as carry_kernel's
  if (nseg <= 0) return hipSuccess;
  if (nseg > kMaxSegs) return hipErrorInvalidValue;
  SegArgs args;
  uint64_t tiles = 0;
  bool vec = true;
  int k = 0;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].len == 0) continue;
    args.a[k] = segs[i].a;
    args.b[k] = segs[i].b;
    args.dst[k] = segs[i].dst;
    args.dst2[k] = DF ? nullptr : segs[i].dst2;
    args.len[k] = segs[i].len;
    args.tile0[k] = (uint32_t)tiles;
    tiles += (segs[i].len + kTile - 1) / kTile;
    vec = vec && aligned16(segs[i].a) && aligned16(segs[i].b) && aligned16(segs[i].dst) &&
          (DF || !segs[i].dst2 || aligned16(segs[i].dst2));
    ++k;
  }
  if (k == 0) return hipSuccess;
  if (tiles >= 0xFFFFFFFFull) return hipErrorInvalidValue;
  args.nseg = k;
  args.tile0[k] = (uint32_t)tiles;
  args.lr = 0.0f;
  uint32_t grid = (uint32_t)tiles;
  if (cu_budget > 0) {
    const uint64_t cap = (uint64_t)cu_budget * kWgPerCuBudget;
    if (grid > cap) grid = (uint32_t)cap;
  }
  void* kargs[] = {&args};
  return launch_kernel(vec ? (const void*)carry_kernel<AF, DF, true> : (const void*)carry_kernel<AF, DF, false>,
                       dim3(grid), dim3(kThreads), kargs, stream);
}

uint64_t stream_store_min_bytes() {
  const char* e = getenv("HC_STREAM_STORE_MIN_BYTES");
  if (!e || !*e) return kStreamStoreMinBytes;
  char* end = nullptr;
  const unsigned long long v = strtoull(e, &end, 10);
  return *end == 0 ? (uint64_t)v : kStreamStoreMinBytes;
}

template <int ES, int OP, int POLICY>
hipError_t launch_step_as(const Seg* segs, int nseg, int cu_budget, hipStream_t stream, float lr) {
  constexpr bool kUsesB = OP == kReduce || OP == kSgd || OP == kReduceSend || OP == kSgdSend;
  constexpr bool kSends = OP == kReduceSend || OP == kSgdSend;
  constexpr uint64_t kTile = (uint64_t)kThreads * (16 / ES) * policy_unroll(POLICY);
  SegArgs args;
  uint64_t tiles = 0;
  bool vec = true;
  int k = 0;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i].len == 0) continue;
    args.a[k] = segs[i].a;
    args.b[k] = kUsesB ? segs[i].b : segs[i].a;
    args.dst[k] = segs[i].dst;
    args.dst2[k] = segs[i].dst2;
    if (kSends && !segs[i].dst2) return hipErrorInvalidValue;
    args.len[k] = segs[i].len;
    args.tile0[k] = (uint32_t)tiles;
    tiles += (segs[i].len + kTile - 1) / kTile;
    vec = vec && aligned16(segs[i].a) && aligned16(segs[i].dst) && (!kUsesB || aligned16(segs[i].b)) &&
          (!kSends || aligned16(segs[i].dst2));
    ++k;
  }
  if (k == 0) return hipSuccess;
  if (tiles >= 0xFFFFFFFFull) return hipErrorInvalidValue;
  args.nseg = k;
  args.tile0[k] = (uint32_t)tiles;
  args.lr = lr;
  uint32_t grid = (uint32_t)tiles;
  if (cu_budget > 0) {
    const uint64_t cap = (uint64_t)cu_budget * kWgPerCuBudget;
    if (grid > cap) grid = (uint32_t)cap;
  }
  if (log_enabled()) {
    static const char* const kOpName[] = {"copy", "reduce", "sgd", "sgd_one", "reduce_send", "sgd_send"};
    static const char* const kPolicyName[] = {"cached", "stream", "budget"};
    uint64_t elems = 0;
    for (int i = 0; i < k; ++i) elems += args.len[i];
    log_line("step launch: op=%s elem_bytes=%d policy=%s segments=%d elements=%llu tiles=%llu grid=%u%s", kOpName[OP],
             ES, kPolicyName[POLICY], k, (unsigned long long)elems, (unsigned long long)tiles, grid,
             vec ? "" : " (element path: a pointer is not 16-byte aligned)");
  }
  void* kargs[] = {&args};
  return launch_kernel(vec ? (const void*)step_kernel<ES, OP, true, POLICY>
                           : (const void*)step_kernel<ES, OP, false, POLICY>,
                       dim3(grid), dim3(kThreads), kargs, stream);
}

// One ring step: picks the launch policy (see kPolicyCached) from the CU
// budget and the bytes the launch writes.
template <int ES, int OP>
hipError_t launch_step(const Seg* segs, int nseg, int cu_budget, hipStream_t stream, float lr = 0.0f) {
  constexpr bool kSends = OP == kReduceSend || OP == kSgdSend;
  if (nseg <= 0) return hipSuccess;
  if (nseg > kMaxSegs) return hipErrorInvalidValue;
  if (cu_budget > 0) return launch_step_as<ES, OP, kPolicyBudget>(segs, nseg, cu_budget, stream, lr);
  uint64_t written = 0;
  for (int i = 0; i < nseg; ++i) written += segs[i].len * ES * (kSends ? 2 : 1);
  if (written >= stream_store_min_bytes())
    return launch_step_as<ES, OP, kPolicyStream>(segs, nseg, cu_budget, stream, lr);
  return launch_step_as<ES, OP, kPolicyCached>(segs, nseg, cu_budget, stream, lr);
}

// The whole allreduce in one launch, one chunk per workgroup ("ResCCL:
// Resource-Efficient Scheduling for Collective Communication", section 3:
// data dependencies exist only within one chunk, and a generated kernel
// loops over its work inside the kernel).  The chunk here is one tile (2048
// fp32 or 4096 bf16 elements): chunks of about 1% of the buffer would leave
// only about 100 R chains, too few workgroups for the GPU (measured on
// MI355X for R=4 x 2^20 fp32: 25 us per allreduce against 14 us with tiles).
// Workgroup (j, c) carries tile c of slice j through every hop of the ring
// in the ring's order, with the same reads and writes as the step-per-launch
// schedule:
//   reduce-scatter step s (0..R-2): receiver q = j+2+s reads what its sender
//     q-1 holds (the sender's input at s = 0, else the partial the sender
//     wrote into its output), adds its own input, writes its output; the
//     last step also writes the sum into the next rank's output (that rank's
//     first all-gather copy);
//   all-gather step s (1..R-2): receiver q = j+1+s copies from q-1.
// Each lane keeps the same elements through the hops, so a hop's read of the
// partial the lane itself wrote one hop before needs no barrier; chunks are
// disjoint, so workgroups never wait for one another.  Bits equal the
// step-per-launch schedule's: the same hop on the same operands in the same
// order.
struct ChainArgs {
  const void* send[kMaxRanks];
  void* recv[kMaxRanks];
  uint64_t count;   // elements per rank
  uint64_t slice;   // slice length (the last slices may be short or empty)
  uint64_t chunk;   // elements per chain: one tile
  uint32_t R;
  uint32_t chains;  // chains per slice
};

template <int ES, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs args) {
  constexpr int V = 16 / ES;
  constexpr int U = 2;
  constexpr uint64_t kTile = (uint64_t)kThreads * V * U;
  const uint32_t R = args.R, tid = threadIdx.x;
  const uint32_t total = R * args.chains;
  for (uint32_t w = blockIdx.x; w < total; w += gridDim.x) {
    const uint32_t j = w / args.chains, c = w % args.chains;
    const uint64_t s0 = (uint64_t)j * args.slice;
    const uint64_t s1 = s0 + args.slice < args.count ? s0 + args.slice : args.count;
    const uint64_t lo = s0 + (uint64_t)c * args.chunk;
    if (s0 >= args.count || lo >= s1) continue;
    const uint64_t hi = lo + args.chunk < s1 ? lo + args.chunk : s1;
    for (uint64_t base = lo; base < hi; base += kTile) {
      if (VEC && base + kTile <= hi) {
        uint4 a[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          a[u] = ld_stream<HC_RING_NT_A>(static_cast<const char*>(args.send[(j + 1) % R]) +
                                         (base + (uint64_t)(u * kThreads + tid) * V) * ES);
        for (uint32_t s = 0; s + 1 < R; ++s) {
          const uint32_t q = (j + 2 + s) % R;
          const char* pb = static_cast<const char*>(args.send[q]);
          char* pd = static_cast<char*>(args.recv[q]);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint64_t off = (base + (uint64_t)(u * kThreads + tid) * V) * ES;
            const uint4 r = vec_hop<ES>(a[u], ld_stream<HC_RING_NT_B>(pb + off));
            st_stream<false>(pd + off, r);
            if (s + 2 == R) st_stream<false>(static_cast<char*>(args.recv[(q + 1) % R]) + off, r);
          }
          if (s + 2 < R) {
#pragma unroll
            for (int u = 0; u < U; ++u) a[u] = ld16(pd + (base + (uint64_t)(u * kThreads + tid) * V) * ES);
          }
        }
        for (uint32_t s = 1; s + 1 < R; ++s) {
          const char* pa = static_cast<const char*>(args.recv[(j + s) % R]);
          char* pd = static_cast<char*>(args.recv[(j + 1 + s) % R]);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint64_t off = (base + (uint64_t)(u * kThreads + tid) * V) * ES;
            st_stream<false>(pd + off, ld16(pa + off));
          }
        }
      } else {
        const uint64_t end = base + kTile < hi ? base + kTile : hi;
        for (uint64_t i = base + tid; i < end; i += kThreads) {
          uint32_t x = ld_elem<ES>(static_cast<const char*>(args.send[(j + 1) % R]), i);
          for (uint32_t s = 0; s + 1 < R; ++s) {
            const uint32_t q = (j + 2 + s) % R;
            char* pd = static_cast<char*>(args.recv[q]);
            const uint32_t r = scalar_hop<ES>(x, ld_elem<ES>(static_cast<const char*>(args.send[q]), i));
            st_elem<ES>(pd, i, r);
            if (s + 2 == R) st_elem<ES>(static_cast<char*>(args.recv[(q + 1) % R]), i, r);
            if (s + 2 < R) x = ld_elem<ES>(pd, i);
          }
          for (uint32_t s = 1; s + 1 < R; ++s)
            st_elem<ES>(static_cast<char*>(args.recv[(j + 1 + s) % R]), i,
                        ld_elem<ES>(static_cast<const char*>(args.recv[(j + s) % R]), i));
        }
      }
    }
  }
}

// Where each workgroup runs: word 2w = its HW_ID register (CU, shader array
// and shader engine fields among others), word 2w + 1 = its XCC_ID (the XCD).
// Each workgroup first holds its CU for hold_ticks of the 100 MHz real-time
// clock (a bounded wait), so that the workgroups of one launch are resident
// together and spread over every CU the stream may use.
__global__ __launch_bounds__(64) void cu_census_kernel(uint32_t* ids, uint32_t hold_ticks) {
  uint32_t hw, xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < hold_ticks) __builtin_amdgcn_s_sleep(8);
  if (threadIdx.x == 0) {
    ids[2 * blockIdx.x] = hw;
    ids[2 * blockIdx.x + 1] = xcc;
  }
}

}  // namespace

hipError_t launch_cu_census(uint32_t* ids, uint32_t n_workgroups, uint32_t hold_us, hipStream_t stream) {
  hipLaunchKernelGGL(cu_census_kernel, dim3(n_workgroups), dim3(64), 0, stream, ids, hold_us * 100u);
  return hipGetLastError();
}

hipError_t launch_reduce_step(const Seg* segs, int nseg, hc_dtype_t dtype, int cu_budget,
                              hipStream_t stream) {
  if (dtype == HC_F32) return launch_step<4, kReduce>(segs, nseg, cu_budget, stream);
  return launch_step<2, kReduce>(segs, nseg, cu_budget, stream);
}

hipError_t launch_reduce_send_step(const Seg* segs, int nseg, hc_dtype_t dtype, int cu_budget, hipStream_t stream) {
  if (dtype == HC_F32) return launch_step<4, kReduceSend>(segs, nseg, cu_budget, stream);
  return launch_step<2, kReduceSend>(segs, nseg, cu_budget, stream);
}

hipError_t launch_sgd_step(const Seg* segs, int nseg, hc_dtype_t dtype, float lr, int cu_budget,
                           hipStream_t stream) {
  const bool one = nseg > 0 && segs[0].b == nullptr;
  const bool send = nseg > 0 && segs[0].dst2 != nullptr;
  if (send && !one)
    return dtype == HC_F32 ? launch_step<4, kSgdSend>(segs, nseg, cu_budget, stream, lr)
                           : launch_step<2, kSgdSend>(segs, nseg, cu_budget, stream, lr);
  if (dtype == HC_F32)
    return one ? launch_step<4, kSgdOne>(segs, nseg, cu_budget, stream, lr)
               : launch_step<4, kSgd>(segs, nseg, cu_budget, stream, lr);
  return one ? launch_step<2, kSgdOne>(segs, nseg, cu_budget, stream, lr)
             : launch_step<2, kSgd>(segs, nseg, cu_budget, stream, lr);
}

hipError_t launch_carry_step(const Seg* segs, int nseg, bool a_f32, bool dst_f32, int cu_budget,
                             hipStream_t stream) {
  if (a_f32) return dst_f32 ? launch_carry<true, true>(segs, nseg, cu_budget, stream)
                            : launch_carry<true, false>(segs, nseg, cu_budget, stream);
  return dst_f32 ? launch_carry<false, true>(segs, nseg, cu_budget, stream)
                 : launch_carry<false, false>(segs, nseg, cu_budget, stream);
}

hipError_t launch_chain_allreduce(void* const* send, void* const* recv, size_t count, size_t es, int R,
                                  int cu_budget, hipStream_t stream) {
  if (R < 2 || R > kMaxRanks || count == 0) return hipErrorInvalidValue;
  const uint64_t tile = (uint64_t)kThreads * (16 / es) * 2;
  ChainArgs args;
  bool vec = true;
  for (int r = 0; r < R; ++r) {
    args.send[r] = send[r];
    args.recv[r] = recv[r];
    vec = vec && aligned16(send[r]) && aligned16(recv[r]);
  }
  args.count = count;
  args.slice = (count + R - 1) / R;
  vec = vec && (args.slice * es) % 16 == 0;           // every slice starts on a 16-byte boundary
  args.chunk = tile;
  args.R = (uint32_t)R;
  const uint64_t chains = (args.slice + args.chunk - 1) / args.chunk;
  if (chains * (uint64_t)R >= 0xFFFFFFFFull) return hipErrorInvalidValue;
  args.chains = (uint32_t)chains;
  uint32_t grid = (uint32_t)(chains * R);
  if (cu_budget > 0) {
    const uint64_t cap = (uint64_t)cu_budget * kWgPerCuBudget;
    if (grid > cap) grid = (uint32_t)cap;
  }
  if (log_enabled())
    log_line("chain launch: elem_bytes=%zu ranks=%d slice=%llu chunk=%llu chains=%u grid=%u%s", es, R,
             (unsigned long long)args.slice, (unsigned long long)args.chunk, args.chains * args.R, grid,
             vec ? "" : " (element path: a pointer or slice start is not 16-byte aligned)");
  void* kargs[] = {&args};
  const void* fn = es == 4 ? (vec ? (const void*)chain_kernel<4, true> : (const void*)chain_kernel<4, false>)
                           : (vec ? (const void*)chain_kernel<2, true> : (const void*)chain_kernel<2, false>);
  return launch_kernel(fn, dim3(grid), dim3(kThreads), kargs, stream);
}

hipError_t launch_copy_step(const Seg* segs, int nseg, size_t elem_bytes, int cu_budget,
                            hipStream_t stream) {
  if (elem_bytes == 4) return launch_step<4, kCopy>(segs, nseg, cu_budget, stream);
  return launch_step<2, kCopy>(segs, nseg, cu_budget, stream);
}

}  // namespace hc
