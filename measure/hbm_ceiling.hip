// hbm_ceiling -- what plain streaming kernels reach on this GPU's HBM for the
// access mixes of the ring hops, at the hops' own operand size and tiling.
//
// The published HBM figure is a peak that no kernel reaches; the useful bar for
// a ring hop is the best a kernel with nothing but the same memory traffic
// achieves.  Three mixes, each a bounded loop over uint4 (16-byte) elements,
// 256 lanes per workgroup, two 16-byte vectors per lane and operand,
// non-temporal loads and ordinary stores (the tiling the ring step kernel
// uses), one tile per workgroup:
//   add    c = a + b (integer lanes): two reads, one write -- a reduce hop;
//   copy   c = a: one read, one write -- an all-gather copy hop;
//   read   two reads folded into a register, no store -- the read side alone.
// Each kernel is timed by its own start and end stamps (hipExtLaunchKernel
// events), mean of `reps` launches after two warm-ups.
//
//   hbm_ceiling [operand_MiB] [reps]   default 128 MiB (one R=8 x 2^26 bf16
//                                      ring step per operand) and 10; prints
//                                      one JSON object.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdio>
#include <cstdlib>

namespace {

#define CK(x)                                                                  \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

constexpr int kLanes = 256, kVec = 2;
constexpr size_t kTile = (size_t)kLanes * kVec;   // uint4 elements per workgroup

__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  uint4 v;
  v.x = __builtin_nontemporal_load(&p->x);
  v.y = __builtin_nontemporal_load(&p->y);
  v.z = __builtin_nontemporal_load(&p->z);
  v.w = __builtin_nontemporal_load(&p->w);
  return v;
}

__device__ __forceinline__ uint4 add4(uint4 a, uint4 b) {
  return make_uint4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__global__ __launch_bounds__(kLanes) void add_kernel(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                     uint4* __restrict__ c, size_t n) {
  const size_t base = blockIdx.x * kTile + threadIdx.x;
  uint4 va[kVec], vb[kVec];
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const size_t i = base + (size_t)u * kLanes;
    if (i < n) {
      va[u] = ld_nt(a + i);
      vb[u] = ld_nt(b + i);
    }
  }
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const size_t i = base + (size_t)u * kLanes;
    if (i < n) c[i] = add4(va[u], vb[u]);
  }
}

__global__ __launch_bounds__(kLanes) void copy_kernel(const uint4* __restrict__ a, uint4* __restrict__ c, size_t n) {
  const size_t base = blockIdx.x * kTile + threadIdx.x;
  uint4 va[kVec];
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const size_t i = base + (size_t)u * kLanes;
    if (i < n) va[u] = ld_nt(a + i);
  }
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const size_t i = base + (size_t)u * kLanes;
    if (i < n) c[i] = va[u];
  }
}

// The folded value is stored only when it equals a pattern the inputs (bytes
// 0x01 and 0x02) cannot produce, so the loads stay live and nothing is
// written; `sink` has one slot per lane of the grid.
__global__ __launch_bounds__(kLanes) void read_kernel(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                      uint4* __restrict__ sink, size_t n) {
  const size_t base = blockIdx.x * kTile + threadIdx.x;
  uint4 acc = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const size_t i = base + (size_t)u * kLanes;
    if (i < n) acc = add4(acc, add4(ld_nt(a + i), ld_nt(b + i)));
  }
  if (acc.x == 1u && acc.y == 2u && acc.z == 3u && acc.w == 4u) sink[blockIdx.x * (size_t)kLanes + threadIdx.x] = acc;
}

}  // namespace

int main(int argc, char** argv) {
  const long mib = argc > 1 ? atol(argv[1]) : 128;
  const int reps = argc > 2 ? atoi(argv[2]) : 10;
  if (mib < 1 || mib > 8192 || reps < 1 || reps > 1000) {
    fprintf(stderr, "usage: hbm_ceiling [operand_MiB 1..8192] [reps 1..1000]\n");
    return 2;
  }
  const size_t bytes = (size_t)mib << 20, n = bytes / 16;
  const unsigned grid = (unsigned)((n + kTile - 1) / kTile);
  uint4 *a, *b, *c, *sink;
  CK(hipMalloc(&a, bytes));
  CK(hipMalloc(&b, bytes));
  CK(hipMalloc(&c, bytes));
  CK(hipMalloc(&sink, (size_t)grid * kLanes * sizeof(uint4)));
  CK(hipMemset(a, 1, bytes));
  CK(hipMemset(b, 2, bytes));
  CK(hipMemset(c, 0, bytes));
  hipStream_t s;
  CK(hipStreamCreate(&s));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));

  size_t nn = n;
  const uint4 *pa = a, *pb = b;
  uint4 *pc = c, *pk = sink;
  void* add_args[] = {&pa, &pb, &pc, &nn};
  void* copy_args[] = {&pa, &pc, &nn};
  void* read_args[] = {&pa, &pb, &pk, &nn};
  struct Mix {
    const char* name;
    const void* fn;
    void** args;
    double bytes;
  } mixes[] = {{"add", (const void*)add_kernel, add_args, 3.0 * bytes},
               {"copy", (const void*)copy_kernel, copy_args, 2.0 * bytes},
               {"read", (const void*)read_kernel, read_args, 2.0 * bytes}};

  printf("{\"operand_bytes\": %zu, \"reps\": %d, \"tiling\": \"256 lanes x 2 x 16 B per operand, one tile per "
         "workgroup, non-temporal loads\", \"peak_gbps\": 8000.0",
         bytes, reps);
  for (const Mix& m : mixes) {
    float total = 0;
    for (int r = 0; r < reps + 2; ++r) {
      CK(hipExtLaunchKernel(m.fn, dim3(grid), dim3(kLanes), m.args, 0, s, e0, e1, 0));
      CK(hipStreamSynchronize(s));
      float ms;
      CK(hipEventElapsedTime(&ms, e0, e1));
      if (r >= 2) total += ms;
    }
    const double us = total * 1000.0 / reps, gbps = m.bytes / us / 1e3;
    printf(", \"%s\": {\"bytes\": %.0f, \"us\": %.2f, \"gbps\": %.1f, \"frac_of_peak\": %.4f}", m.name, m.bytes, us,
           gbps, gbps / 8000.0);
  }
  printf("}\n");
  CK(hipFree(a));
  CK(hipFree(b));
  CK(hipFree(c));
  CK(hipFree(sink));
  return 0;
}
