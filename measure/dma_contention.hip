// dma_contention -- the all-gather copy offload measured in a process of its
// own, linked against the system ROCm runtime.
//
// "HOCCL: Offloading Collective Communication from GPU Cores to Accelerate
// Distributed Training" (section 2) moves collective copies off the GPU cores
// so that they stop contending with compute kernels; a reduction cannot move.
// libhc's hc_opts_t.copy_engine = 1 runs all-gather copy steps as
// hipMemcpyDeviceToDeviceNoCU copies.  Whether a HIP runtime honours that
// kind is the runtime's choice: the one in /opt/rocm hands them to the DMA
// engines, the one bundled with the PyTorch wheel runs them as blit kernels
// on the compute units.  This program therefore runs outside any torch
// process, with the GEMM from rocBLAS.
//
//   dma_contention verify [dir]
//                           small all-gather (R=8 x 65,540 bf16): the
//                           copy-engine output must equal the copy-kernel
//                           output byte for byte (with dir: the inputs and the
//                           oracle's expected output read from dir, see
//                           verify_against), and the copy-engine run must
//                           finish while a bounded spin kernel holds every
//                           wave slot of the GPU.  Exit 0 when both hold.
//   dma_contention bench    R=8 slices of 2^25 bf16 -> 8 outputs of 2^28
//                           (the all-gather after the reduce-scatter of an
//                           8 x 2^28 bf16 allreduce), on copy kernels and on
//                           the DMA engines, alone and beside a loop of
//                           8192^3 bf16 GEMMs; prints one JSON object.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "hc.h"

namespace {

#define CK(x)                                                                              \
  do {                                                                                     \
    hipError_t e_ = (x);                                                                   \
    if (e_ != hipSuccess) {                                                                \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);  \
      std::exit(2);                                                                        \
    }                                                                                      \
  } while (0)
#define CKB(x)                                                                       \
  do {                                                                               \
    rocblas_status s_ = (x);                                                         \
    if (s_ != rocblas_status_success) {                                              \
      std::fprintf(stderr, "rocBLAS status %d at line %d\n", (int)s_, __LINE__);    \
      std::exit(2);                                                                  \
    }                                                                                \
  } while (0)
#define CKH(x)                                                                          \
  do {                                                                                  \
    hc_status_t h_ = (x);                                                               \
    if (h_ != HC_SUCCESS) {                                                             \
      std::fprintf(stderr, "hc status %d: %s at line %d\n", (int)h_, hc_last_error(), __LINE__); \
      std::exit(2);                                                                     \
    }                                                                                   \
  } while (0)

constexpr int kN = 256;  // neutral stand-in when the CU count query fails

// Deterministic bf16 fill: a small normal-range value per element (sign,
// exponent 120..127, 7 fraction bits from a hash of the index and the seed).
__global__ void fill_bf16(uint16_t* p, size_t n, uint32_t seed) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    uint32_t h = (uint32_t)i * 0x9E3779B1u ^ seed * 0x85EBCA77u;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    p[i] = (uint16_t)(((h >> 31) << 15) | ((120u + ((h >> 8) & 7u)) << 7) | (h & 0x7Fu));
  }
}

__global__ void count_diff(const uint32_t* a, const uint32_t* b, size_t words, unsigned long long* bad) {
  unsigned long long local = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    local += a[i] != b[i];
  if (local) atomicAdd(bad, local);
}

// Holds a wave slot until `ticks` of the 100 MHz realtime counter have passed
// since the wave started: a bounded wait that every wave leaves.
__global__ __launch_bounds__(256) void hold_slots(unsigned long long ticks, int* sink) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long t = t0;
  int n = 0;
  while (t - t0 < ticks) {
    t = __builtin_amdgcn_s_memrealtime();
    ++n;
  }
  if (n == -1) sink[0] = n;
}

double now_ms() {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

std::string runtime_path() {
  FILE* f = std::fopen("/proc/self/maps", "r");
  if (!f) return "unknown";
  char line[4096];
  std::string found = "unknown";
  while (std::fgets(line, sizeof line, f)) {
    const char* p = std::strstr(line, "libamdhip64");
    if (!p) continue;
    const char* s = std::strchr(line, '/');
    if (!s) continue;
    found.assign(s);
    while (!found.empty() && (found.back() == '\n' || found.back() == ' ')) found.pop_back();
    break;
  }
  std::fclose(f);
  return found;
}

struct Ring {
  int R;
  size_t L;
  std::vector<void*> send, out;
};

Ring make_ring(int R, size_t L) {
  Ring g{R, L, std::vector<void*>(R), std::vector<void*>(R)};
  for (int r = 0; r < R; ++r) {
    CK(hipMalloc(&g.send[r], L * 2));
    CK(hipMalloc(&g.out[r], L * 2 * R));
    hipLaunchKernelGGL(fill_bf16, dim3(1024), dim3(256), 0, 0, static_cast<uint16_t*>(g.send[r]), L, 1000u + r);
    CK(hipGetLastError());
    CK(hipMemset(g.out[r], 0, L * 2 * R));
  }
  CK(hipDeviceSynchronize());
  return g;
}

void free_ring(Ring& g) {
  for (int r = 0; r < g.R; ++r) {
    CK(hipFree(g.send[r]));
    CK(hipFree(g.out[r]));
  }
}

void all_gather(Ring& g, int engine, hipStream_t s) {
  hc_opts_t o = {};
  o.copy_engine = engine;
  CKH(hc_all_gather(g.send.data(), g.out.data(), g.L, HC_BF16, g.R, &o, s));
}

// Runs the copy-engine all-gather on stream B while every wave slot is held
// for `hold_ms`; returns true when it completed well before the slots were
// released.  The runtime picks the engine per stream, so B is the stream the
// measured copies use.
bool finishes_during_hold(Ring& g, hipStream_t B, double hold_ms, double* t_ag, double* t_hold) {
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || ncu <= 0) ncu = kN;
  int* sink;
  CK(hipMalloc(&sink, 4));
  hipStream_t A;
  CK(hipStreamCreateWithFlags(&A, hipStreamNonBlocking));
  hipEvent_t held, done;
  CK(hipEventCreate(&held));
  CK(hipEventCreate(&done));
  CK(hipDeviceSynchronize());
  const double t0 = now_ms();
  // 8 workgroups of 4 waves per CU: 32 waves, every slot of a CU.
  hipLaunchKernelGGL(hold_slots, dim3(ncu * 8), dim3(256), 0, A, (unsigned long long)(hold_ms * 1e5), sink);
  CK(hipGetLastError());
  CK(hipEventRecord(held, A));
  while (now_ms() - t0 < 2.0) {
  }
  all_gather(g, 1, B);
  CK(hipEventRecord(done, B));
  CK(hipEventSynchronize(done));
  *t_ag = now_ms() - t0;
  CK(hipEventSynchronize(held));
  *t_hold = now_ms() - t0;
  CK(hipEventDestroy(held));
  CK(hipEventDestroy(done));
  CK(hipStreamDestroy(A));
  CK(hipFree(sink));
  return *t_ag < *t_hold - 0.1 * hold_ms;
}

unsigned long long compare_outputs(Ring& a, Ring& b) {
  unsigned long long* bad;
  CK(hipMalloc(&bad, 8));
  CK(hipMemset(bad, 0, 8));
  for (int r = 0; r < a.R; ++r)
    hipLaunchKernelGGL(count_diff, dim3(1024), dim3(256), 0, 0, static_cast<const uint32_t*>(a.out[r]),
                       static_cast<const uint32_t*>(b.out[r]), a.L * a.R * 2 / 4, bad);
  CK(hipGetLastError());
  unsigned long long h = 0;
  CK(hipMemcpy(&h, bad, 8, hipMemcpyDeviceToHost));
  CK(hipFree(bad));
  return h;
}

// Reads a whole file into a vector; false when it cannot.
bool read_file(const std::string& path, std::vector<uint16_t>& out, size_t words) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  out.resize(words);
  const size_t got = std::fread(out.data(), 2, words, f);
  std::fclose(f);
  return got == words;
}

// verify with inputs and the expected all-gather from a directory written by
// the test (the oracle's result): meta.txt "R L", in_<r>.bin (L bf16 words),
// expected_<r>.bin (R * L words).  Returns the mismatched words of the
// copy-engine all-gather against the expected bytes, or -1 on a bad input.
long long verify_against(const char* dir, int* R_out, size_t* L_out, Ring* ring) {
  int R = 0;
  size_t L = 0;
  {
    FILE* f = std::fopen((std::string(dir) + "/meta.txt").c_str(), "r");
    if (!f) return -1;
    const int got = std::fscanf(f, "%d %zu", &R, &L);
    std::fclose(f);
    if (got != 2 || R < 1 || R > HC_MAX_RANKS || L < 1 || L > ((size_t)1 << 26)) return -1;
  }
  Ring g = make_ring(R, L);
  std::vector<uint16_t> h;
  for (int r = 0; r < R; ++r) {
    if (!read_file(std::string(dir) + "/in_" + std::to_string(r) + ".bin", h, L)) return -1;
    CK(hipMemcpy(g.send[r], h.data(), L * 2, hipMemcpyHostToDevice));
  }
  all_gather(g, 1, 0);
  CK(hipDeviceSynchronize());
  long long bad = 0;
  std::vector<uint16_t> got(L * R), want;
  for (int r = 0; r < R; ++r) {
    if (!read_file(std::string(dir) + "/expected_" + std::to_string(r) + ".bin", want, L * R)) return -1;
    CK(hipMemcpy(got.data(), g.out[r], L * R * 2, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < L * R; ++i) bad += got[i] != want[i];
  }
  *R_out = R;
  *L_out = L;
  *ring = g;
  return bad;
}

int verify(const char* dir) {
  if (dir) {   // the copy-engine all-gather against the oracle's bytes, then the offload check on the same ring
    int R = 0;
    size_t L = 0;
    Ring g;
    const long long bad = verify_against(dir, &R, &L, &g);
    if (bad < 0) {
      std::fprintf(stderr, "verify: cannot read the inputs in %s\n", dir);
      return 2;
    }
    double t_ag = 0, t_hold = 0;
    hipStream_t B;
    CK(hipStreamCreateWithFlags(&B, hipStreamNonBlocking));
    const bool offloaded = finishes_during_hold(g, B, 200.0, &t_ag, &t_hold);
    CK(hipStreamDestroy(B));
    std::printf("{\"mode\": \"verify\", \"against\": \"expected files\", \"ranks\": %d, \"slice\": %zu, "
                "\"mismatched_words\": %lld, \"copy_engine_done_ms\": %.2f, \"slots_released_ms\": %.2f, "
                "\"no_compute_units\": %s, \"hip_runtime\": \"%s\"}\n",
                R, L, bad, t_ag, t_hold, offloaded ? "true" : "false", runtime_path().c_str());
    free_ring(g);
    return bad == 0 && offloaded ? 0 : 1;
  }
  const int R = 8;
  const size_t L = 65536 + 4;  // even: the comparison reads whole words
  Ring cu = make_ring(R, L), dma = make_ring(R, L);
  all_gather(cu, 0, 0);
  all_gather(dma, 1, 0);
  CK(hipDeviceSynchronize());
  const unsigned long long bad = compare_outputs(cu, dma);
  double t_ag = 0, t_hold = 0;
  hipStream_t B;
  CK(hipStreamCreateWithFlags(&B, hipStreamNonBlocking));
  const bool offloaded = finishes_during_hold(dma, B, 200.0, &t_ag, &t_hold);
  CK(hipStreamDestroy(B));
  std::printf("{\"mode\": \"verify\", \"ranks\": %d, \"slice\": %zu, \"mismatched_words\": %llu, "
              "\"copy_engine_done_ms\": %.2f, \"slots_released_ms\": %.2f, \"no_compute_units\": %s, "
              "\"hip_runtime\": \"%s\"}\n",
              R, L, bad, t_ag, t_hold, offloaded ? "true" : "false", runtime_path().c_str());
  free_ring(cu);
  free_ring(dma);
  return bad == 0 && offloaded ? 0 : 1;
}

double median(std::vector<double> v) {
  if (v.empty()) return 0.0;
  std::sort(v.begin(), v.end());
  const size_t n = v.size();
  return n % 2 ? v[n / 2] : 0.5 * (v[n / 2 - 1] + v[n / 2]);
}

int bench() {
  const int R = 8, M = 8192;
  const size_t L = (size_t)1 << 25;
  Ring g = make_ring(R, L);
  void *A, *B, *C;
  CK(hipMalloc(&A, (size_t)M * M * 2));
  CK(hipMalloc(&B, (size_t)M * M * 2));
  CK(hipMalloc(&C, (size_t)M * M * 2));
  hipLaunchKernelGGL(fill_bf16, dim3(1024), dim3(256), 0, 0, static_cast<uint16_t*>(A), (size_t)M * M, 1u);
  hipLaunchKernelGGL(fill_bf16, dim3(1024), dim3(256), 0, 0, static_cast<uint16_t*>(B), (size_t)M * M, 2u);
  CK(hipGetLastError());
  hipStream_t main_s, side;
  CK(hipStreamCreateWithFlags(&main_s, hipStreamNonBlocking));
  CK(hipStreamCreateWithFlags(&side, hipStreamNonBlocking));
  rocblas_handle h;
  CKB(rocblas_create_handle(&h));
  CKB(rocblas_set_stream(h, main_s));
  const float alpha = 1.0f, beta = 0.0f;
  auto gemm = [&]() {
    CKB(rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, M, M, M, &alpha, A,
                        rocblas_datatype_bf16_r, M, B, rocblas_datatype_bf16_r, M, &beta, C, rocblas_datatype_bf16_r,
                        M, C, rocblas_datatype_bf16_r, M, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0));
  };
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  for (int i = 0; i < 3; ++i) gemm();
  CK(hipDeviceSynchronize());
  CK(hipEventRecord(e0, main_s));
  for (int i = 0; i < 10; ++i) gemm();
  CK(hipEventRecord(e1, main_s));
  CK(hipEventSynchronize(e1));
  float ms = 0;
  CK(hipEventElapsedTime(&ms, e0, e1));
  const double t_gemm0 = ms / 10.0;
  const double ag_bytes = 2.0 * 2.0 * (double)L * R * R;  // every output element read once and written once
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || ncu <= 0) ncu = kN;
  double t_ag = 0, t_hold = 0;
  all_gather(g, 1, side);  // warm the copy-engine path of this stream
  CK(hipDeviceSynchronize());
  const bool offloaded = finishes_during_hold(g, side, 200.0, &t_ag, &t_hold);

  std::string rows;
  for (int engine = 0; engine < 2; ++engine) {
    for (int i = 0; i < 2; ++i) all_gather(g, engine, side);
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(e0, side));
    all_gather(g, engine, side);
    CK(hipEventRecord(e1, side));
    CK(hipEventSynchronize(e1));
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double t_alone = ms;
    // the GEMM alone again right before the concurrent run, so that both
    // figures come from the same clock and thermal state
    CK(hipEventRecord(e0, main_s));
    for (int i = 0; i < 20; ++i) gemm();
    CK(hipEventRecord(e1, main_s));
    CK(hipEventSynchronize(e1));
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double t_gemm = ms / 20.0;
    // concurrent: GEMMs on the main stream for as long as the all-gather runs
    const int iters = std::max(4, (int)(t_alone / t_gemm) + 2);
    std::vector<hipEvent_t> ge(iters + 1);
    for (auto& e : ge) CK(hipEventCreate(&e));
    hipEvent_t base, r0, r1;
    CK(hipEventCreate(&base));
    CK(hipEventCreate(&r0));
    CK(hipEventCreate(&r1));
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(base, main_s));
    CK(hipStreamWaitEvent(side, base, 0));
    CK(hipEventRecord(r0, side));
    all_gather(g, engine, side);
    CK(hipEventRecord(r1, side));
    CK(hipEventRecord(ge[0], main_s));
    for (int i = 0; i < iters; ++i) {
      gemm();
      CK(hipEventRecord(ge[i + 1], main_s));
    }
    CK(hipDeviceSynchronize());
    std::vector<double> gt(iters + 1);
    for (int i = 0; i <= iters; ++i) {
      CK(hipEventElapsedTime(&ms, base, ge[i]));
      gt[i] = ms;
    }
    float a0, a1;
    CK(hipEventElapsedTime(&a0, base, r0));
    CK(hipEventElapsedTime(&a1, base, r1));
    std::vector<double> overl;
    double num = 0, den = 0;
    const double cu_used = engine ? 0.0 : (double)ncu;
    for (int i = 0; i < iters; ++i) {
      if (gt[i] < a1 && gt[i + 1] > a0) overl.push_back(gt[i + 1] - gt[i]);
      const double lo = std::max(gt[i], (double)a0), hi = std::min(gt[i + 1], (double)a1);
      den += gt[i + 1] - gt[i];
      if (hi > lo) num += (hi - lo) * cu_used / ncu;
    }
    const double t_conc = median(overl);
    char buf[1024];
    std::snprintf(buf, sizeof buf,
                  "%s{\"op\": \"all_gather\", \"copies_on\": \"%s\", \"ag_alone_ms\": %.4f, \"ag_concurrent_ms\": %.4f, "
                  "\"ag_alone_gbps\": %.1f, \"ag_concurrent_gbps\": %.1f, \"gemm_alone_ms\": %.4f, "
                  "\"gemm_concurrent_ms\": %.4f, \"gemm_slowdown\": %.4f, \"contention_rate\": %.5f}",
                  rows.empty() ? "" : ", ", engine ? "dma_engines" : "cu_kernels", t_alone, (double)(a1 - a0),
                  ag_bytes / t_alone / 1e6, ag_bytes / (a1 - a0) / 1e6, t_gemm, t_conc, t_conc / t_gemm - 1.0,
                  den > 0 ? num / den : 0.0);
    rows += buf;
    for (auto& e : ge) CK(hipEventDestroy(e));
    CK(hipEventDestroy(base));
    CK(hipEventDestroy(r0));
    CK(hipEventDestroy(r1));
  }
  std::printf("{\"mode\": \"bench\", \"ranks\": %d, \"slice\": %zu, \"gemm_tflops_alone\": %.1f, "
              "\"copy_engine_without_compute_units\": %s, \"copy_engine_done_ms_while_slots_held\": %.2f, "
              "\"slots_released_ms\": %.2f, \"hip_runtime\": \"%s\", \"rows\": [%s]}\n",
              R, L, 2.0 * M * (double)M * M / (t_gemm0 / 1e3) / 1e12, offloaded ? "true" : "false",
              t_ag, t_hold, runtime_path().c_str(), rows.c_str());
  CKB(rocblas_destroy_handle(h));
  CK(hipFree(A));
  CK(hipFree(B));
  CK(hipFree(C));
  free_ring(g);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  const char* mode = argc > 1 ? argv[1] : "verify";
  if (!std::strcmp(mode, "verify")) return verify(argc > 2 ? argv[2] : nullptr);
  if (!std::strcmp(mode, "bench")) return bench();
  std::fprintf(stderr, "usage: dma_contention verify|bench\n");
  return 2;
}
