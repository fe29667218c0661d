// codec_kernels.hip -- HCZ1 compress / decompress and the fused compressed
// ring allreduce, for gfx950.
//
// compress: one workgroup per 32 KB block, block = workgroup index.  A block
// publishes its record size as soon as it has chosen its code length, then
// encodes into LDS, then looks back over its predecessors' published sizes
// for its byte offset (a decoupled look-back scan) and writes the record
// straight into the final stream: one read of the input, one write of the
// output, no temporary buffers and no coalescing pass ("CCCL: In-GPU
// Compression-Coupled Collective Communication", section 4.4).  The
// look-back waits only on lower-indexed blocks, and every wait is bounded
// (lookback.hpp says why the waits end).
//
// decompress: one workgroup per block; every block validates the stream
// header and its own record before it reads it; reads never leave in_bytes.
//
// compressed ring allreduce: "CCCL ...", section 5 (selective compression):
// the sender compresses what it sends, the receiver decompresses it, reduces
// with its own uncompressed data and compresses the result for the next hop;
// the fused kernel does decompress -> hop -> compress per block in one pass
// with the block's values in registers.  Wire records sit in fixed-size
// slots, one per block (the preallocated regions of section 4.4).
#include <stdlib.h>

#include <mutex>

#include "car.hpp"
#include "codec.hpp"
#include "launch.hpp"
#include "lookback.hpp"
#include "schedule.hpp"

// Static scratch of the allocation-free compress entry point: the look-back
// head and one descriptor per block for up to kNoAllocMaxBlocks blocks.  Each
// GPU the library runs on holds its own copy until the process ends.  Host
// code never passes this name to a kernel (on the host it is a stand-in, not
// a device address): it takes each device's address once, through
// hipGetSymbolAddress, and passes that.
static __device__ __align__(256) uint8_t scratch[hc::kNoAllocScratchBytes];

namespace hc {

using namespace codec;

namespace {

// Shared-table pieces of the table-scope variant, laid out after the
// look-back workspace (worst case: one group per block).
struct ScopeWs {
  uint32_t* ghist;                 // [groups][256] summed exponent counts
  uint16_t* bhist;                 // [full blocks][256] each block's counts
  uint8_t* order;                  // [groups][256] rank -> exponent
  uint32_t* gb;                    // [groups] chosen b
  uint32_t* esc;                   // [full blocks][8] escapes per b (index b, 1..7)
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Byte offsets of the ScopeWs arrays after a base of `base` bytes, for
// `groups` groups and `full` full blocks; returns the end.
size_t scope_layout(size_t base, size_t groups, size_t full, size_t (&off)[5]) {
  size_t o = align256(base);
  off[0] = o; o = align256(o + groups * 256 * 4);
  off[1] = o; o = align256(o + full * 256 * 2);
  off[2] = o; o = align256(o + groups * 256);
  off[3] = o; o = align256(o + groups * 4);
  off[4] = o; o = align256(o + full * 8 * 4);
  return o;
}

constexpr uint32_t kSumChunk = 64;  // blocks one workgroup adds into a group histogram (at least)


__global__ void fill_u32_kernel(uint32_t* dst, uint32_t value, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = value;
}

__global__ void set_u64_kernel(uint64_t* dst, uint64_t value) { *dst = value; }

// Validates a stream that holds no elements: just the 32-byte header.
__global__ void check_empty_stream_kernel(const uint8_t* in, uint64_t in_bytes, uint32_t magic, int32_t* status) {
  bool ok = in_bytes >= 32;
  if (ok) {
    const uint32_t* h = reinterpret_cast<const uint32_t*>(in);
    ok = h[0] == magic && h[1] == kB && *reinterpret_cast<const uint64_t*>(in + 8) == 0 && h[4] == 0 &&
         h[5] == 0 && *reinterpret_cast<const uint64_t*>(in + 24) == 32;
  }
  if (!ok) *status = HC_ERR_CORRUPT_STREAM;
}

__global__ void empty_stream_kernel(uint8_t* out, uint32_t magic, uint64_t* out_bytes) {
  write_stream_header(out, magic, kB, 0, 0, 32);
  *out_bytes = 32;
}

// SCOPED: the block's code table comes from its group's shared table (sc),
// built by the scope kernels below, instead of its own histogram.
template <bool SCOPED>
__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kCW))) void compress_kernel(
    const uint16_t* __restrict__ in, uint64_t n, uint8_t* __restrict__ out, uint64_t* __restrict__ out_bytes,
    CompressWs* __restrict__ ws, uint32_t nb, ScopeWs sc, uint32_t group, uint32_t spin_limit) {
  __shared__ Smem s;
  const int t = threadIdx.x;
  const uint32_t bid = blockIdx.x;
  const uint64_t first = (uint64_t)bid * kB;
  const uint32_t m = (uint32_t)((n - first) < kB ? (n - first) : kB);
  uint4 v[kPer];
  load_block(in + first, m, v);
  if constexpr (!SCOPED) zero_hist(s);  // while the block is on its way
  __syncthreads();
  Plan p;
  if constexpr (SCOPED) {
    const uint32_t g = bid / group;  // only read for full blocks
    p = m == kB ? given_plan(sc.order + 256ull * g, sc.gb[g], sc.esc[8ull * bid + sc.gb[g]], m, s)
                : given_plan(nullptr, 0, 0, m, s);
  } else {
    p = plan_block<true>(v, m, s);
  }
  if (t == 0) publish(&ws->desc[bid], (bid == 0 ? kFlagIncl : kFlagAgg) | p.rec_bytes);
  write_block(v, p, s);
  if (t < 64) {
    bool ok = true;
    const uint64_t excl = lookback_wave(ws, bid, p.rec_bytes, spin_limit, &ok);
    if (t == 0) {
      s.misc[0] = excl;
      s.misc[1] = ok;
      if (bid != nb - 1) lookback_count_done(ws, bid, ok);
    }
  }
  __syncthreads();
  if (!s.misc[1]) {   // no offset: write nothing; the last block reports no stream
    if (t == 0 && bid == nb - 1) *out_bytes = 0;
    return;
  }
  const uint64_t off = header_bytes(nb) + s.misc[0];
  copy_out(s, out + off, p.rec_bytes);
  if (t == 0) reinterpret_cast<uint64_t*>(out + 32)[bid] = off;
  if (bid == nb - 1 && t < 64) {   // the last block's first wave
    const bool failed = lookback_failed(ws, nb, spin_limit);
    if (t == 0) {
      const uint64_t total = off + p.rec_bytes;
      write_stream_header(out, kMagic, kB, n, nb, total);
      *out_bytes = failed ? 0 : total;
    }
  }
}

// The three-round baseline of "CCCL ...", section 4.4 (compress into
// temporaries, prefix of the sizes, coalescing copy), with the same encoder.
// Round 1: every block encodes into its own fixed-size slot.
__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kCW))) void staged_encode_kernel(
    const uint16_t* __restrict__ in, uint64_t n, uint8_t* __restrict__ slots, uint32_t* __restrict__ sizes) {
  __shared__ Smem s;
  const uint32_t bid = blockIdx.x;
  zero_hist(s);
  __syncthreads();
  const uint64_t first = (uint64_t)bid * kB;
  const uint32_t m = (uint32_t)((n - first) < kB ? (n - first) : kB);
  uint4 v[kPer];
  load_block(in + first, m, v);
  const Plan p = plan_block<true>(v, m, s);
  write_block(v, p, s);
  __syncthreads();
  copy_out(s, slots + (uint64_t)bid * kRawFull, p.rec_bytes);
  if (threadIdx.x == 0) sizes[bid] = p.rec_bytes;
}

// Round 2: byte offset of every record (exclusive prefix of the sizes after
// the stream header and offset table); offs[nb] is the stream size.  One
// workgroup: each thread sums a run of sizes, the 1024 run sums are scanned
// in LDS, and each thread writes its run's offsets.
__global__ __launch_bounds__(1024) void staged_scan_kernel(const uint32_t* __restrict__ sizes, uint32_t nb,
                                                           uint64_t* __restrict__ offs) {
  __shared__ uint64_t part[2][1024];
  const uint32_t t = threadIdx.x;
  const uint32_t per = (nb + 1023u) / 1024u;
  const uint32_t lo = t * per < nb ? t * per : nb, hi = lo + per < nb ? lo + per : nb;
  uint64_t sum = 0;
  for (uint32_t j = lo; j < hi; ++j) sum += sizes[j];
  int cur = 0;
  part[cur][t] = sum;
  __syncthreads();
  for (uint32_t d = 1; d < 1024; d <<= 1) {   // inclusive scan
    const uint64_t x = part[cur][t] + (t >= d ? part[cur][t - d] : 0ull);
    cur ^= 1;
    part[cur][t] = x;
    __syncthreads();
  }
  uint64_t base = header_bytes(nb) + part[cur][t] - sum;
  for (uint32_t j = lo; j < hi; ++j) {
    offs[j] = base;
    base += sizes[j];
  }
  if (t == 1023) offs[nb] = header_bytes(nb) + part[cur][t];
}

// Round 3: every record copied from its slot to its place in the stream.
__global__ __launch_bounds__(256) void staged_copy_kernel(const uint8_t* __restrict__ slots,
                                                          const uint32_t* __restrict__ sizes,
                                                          const uint64_t* __restrict__ offs, uint8_t* __restrict__ out,
                                                          uint64_t n, uint32_t nb, uint64_t* __restrict__ out_bytes) {
  const uint32_t bid = blockIdx.x, t = threadIdx.x;
  const uint32_t n16 = sizes[bid] / 16u;
  const uint64_t off = offs[bid];
  const uint8_t* src = slots + (uint64_t)bid * kRawFull;
  for (uint32_t i = t; i < n16; i += 256) st16(out + off + 16ull * i, ld16(src + 16ull * i));
  if (t == 0) {
    reinterpret_cast<uint64_t*>(out + 32)[bid] = off;
    if (bid == nb - 1) {
      write_stream_header(out, kMagic, kB, n, nb, offs[nb]);
      *out_bytes = offs[nb];
    }
  }
}

// Table scope, step 1: each full block's exponent histogram, one block per
// workgroup.  Workgroup i counts block full - 1 - i: the blocks are read from
// the last one down, so that the encoder, which starts from block 0, finds
// the blocks read last still in the cache.  (Workgroups that each walked 16
// blocks, loading the next while counting the current one, ran 108 us on
// 2^28 elements; one block per workgroup, with the dispatcher overlapping
// workgroups, 103 us.)
__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kCW))) void scope_hist_kernel(
    const uint16_t* __restrict__ in, ScopeWs sc, uint32_t full) {
  __shared__ Smem s;
  const uint32_t t = threadIdx.x;
  const uint32_t k = full - 1u - blockIdx.x;   // the grid covers the full blocks
  uint4 v[kPer];
  load_block(in + (uint64_t)k * kB, kB, v);
  const uint32_t cnt = block_histogram<false>(v, s);   // cnt <= 16384
  if (t < 256u) sc.bhist[256ull * k + t] = (uint16_t)cnt;
}

// Step 2: each group's histogram, `chunk` blocks per workgroup (grid:
// groups x chunks per group), added into the zeroed ghist.
__global__ __launch_bounds__(256) void scope_sum_kernel(ScopeWs sc, uint32_t group, uint32_t full, uint32_t chunk) {
  const uint32_t g = blockIdx.x, t = threadIdx.x;
  const uint64_t g0 = (uint64_t)g * group;
  const uint64_t k0 = g0 + (uint64_t)blockIdx.y * chunk;
  const uint64_t gend = g0 + group < full ? g0 + group : full;
  const uint64_t k1 = k0 + chunk < gend ? k0 + chunk : gend;
  uint32_t sum = 0;
  uint64_t k = k0;
  for (; k + 8u <= k1; k += 8u) {   // eight rows in flight: the loop is latency-bound
    uint32_t x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = sc.bhist[256ull * (k + u) + t];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += x[u];
  }
  for (; k < k1; ++k) sum += sc.bhist[256ull * k + t];
  if (sum) atomicAdd(&sc.ghist[256ull * g + t], sum);
}

// Step 3: each group's symbol order, (count desc, exponent asc).  Exponents
// that never occur rank last in exponent order; the occurring ones (a few
// dozen in practice) are compacted and ranked against each other only.
__global__ __launch_bounds__(256) void scope_rank_kernel(ScopeWs sc) {
  __shared__ unsigned long long key[256];
  __shared__ uint32_t wcount[4];
  const uint32_t g = blockIdx.x, t = threadIdx.x, lane = t & 63u, wave = t >> 6;
  const uint32_t cnt = sc.ghist[256ull * g + t];
  const unsigned long long mine = ((unsigned long long)cnt << 8) | (255u - t);
  const uint64_t nz = __ballot(cnt > 0);
  if (lane == 0) wcount[wave] = (uint32_t)__popcll(nz);
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (uint32_t w = 0; w < 4; ++w) {
    before += w < wave ? wcount[w] : 0u;
    total += wcount[w];
  }
  const uint32_t nz_below = before + (uint32_t)__popcll(nz & ((1ull << lane) - 1ull));
  if (cnt) key[nz_below] = mine;
  __syncthreads();
  uint32_t rank;
  if (cnt) {
    rank = 0;
    for (uint32_t j = 0; j < total; ++j) rank += key[j] > mine;
  } else {
    rank = total + (t - nz_below);
  }
  sc.order[256ull * g + rank] = (uint8_t)t;
}

// Step 4: every full block's escapes for each b under its group's order:
// an inclusive scan of the block's counts in rank order, read at 2^b - 1.
__global__ __launch_bounds__(128) void scope_esc_kernel(ScopeWs sc, uint32_t group) {
  __shared__ uint32_t scan[2][128];
  const uint32_t k = blockIdx.x, t = threadIdx.x, g = k / group;
  uint32_t x = t < 127u ? sc.bhist[256ull * k + sc.order[256ull * g + t]] : 0u;
  int cur = 0;
  scan[cur][t] = x;
  __syncthreads();
#pragma unroll
  for (uint32_t d = 1; d < 128; d <<= 1) {
    x = scan[cur][t] + (t >= d ? scan[cur][t - d] : 0u);
    cur ^= 1;
    scan[cur][t] = x;
    __syncthreads();
  }
  if (t >= 1u && t <= 7u) sc.esc[8ull * k + t] = kB - scan[cur][(1u << t) - 2u];
}

__device__ __forceinline__ uint32_t pick_b(const unsigned long long (&sum)[8]) {
  uint32_t best_b = 1;
#pragma unroll
  for (uint32_t b = 2; b <= 7; ++b)
    if (sum[b] < sum[best_b]) best_b = b;
  return best_b;
}

// Step 5: each group's b, the smallest summed coded size over its blocks,
// ties to the smaller b.  Small groups: one thread per group.
__global__ __launch_bounds__(256) void scope_pick_small_kernel(ScopeWs sc, uint32_t group, uint32_t full,
                                                               uint32_t groups) {
  const uint32_t g = blockIdx.x * 256u + threadIdx.x;
  if (g >= groups) return;
  const uint64_t g0 = (uint64_t)g * group;
  const uint64_t gend = g0 + group < full ? g0 + group : full;
  unsigned long long sum[8] = {};
  for (uint64_t k = g0; k < gend; ++k) {
#pragma unroll
    for (uint32_t b = 1; b <= 7; ++b) sum[b] += coded_bytes(b, sc.esc[8ull * k + b]);
  }
  sc.gb[g] = pick_b(sum);
}

// Large groups: a workgroup per group.
__global__ __launch_bounds__(256) void scope_pick_kernel(ScopeWs sc, uint32_t group, uint32_t full) {
  __shared__ unsigned long long part[4][8];
  const uint32_t g = blockIdx.x, t = threadIdx.x, lane = t & 63u, wave = t >> 6;
  const uint64_t g0 = (uint64_t)g * group;
  const uint64_t gend = g0 + group < full ? g0 + group : full;
  unsigned long long sum[8] = {};
  // a block's escapes as two 16-byte vectors (b = 0..3, 4..7; entry 0 unused)
  const uint4* e4 = reinterpret_cast<const uint4*>(sc.esc);
  auto add = [&](const uint4& lo, const uint4& hi) {
    sum[1] += coded_bytes(1, lo.y);
    sum[2] += coded_bytes(2, lo.z);
    sum[3] += coded_bytes(3, lo.w);
    sum[4] += coded_bytes(4, hi.x);
    sum[5] += coded_bytes(5, hi.y);
    sum[6] += coded_bytes(6, hi.z);
    sum[7] += coded_bytes(7, hi.w);
  };
  uint64_t k = g0 + t;
  for (; k + 768u < gend; k += 1024u) {   // four blocks per thread in flight: the loop is latency-bound
    uint4 lo[4], hi[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      lo[u] = e4[2 * (k + 256u * u)];
      hi[u] = e4[2 * (k + 256u * u) + 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) add(lo[u], hi[u]);
  }
  for (; k < gend; k += 256u) add(e4[2 * k], e4[2 * k + 1]);
#pragma unroll
  for (uint32_t b = 1; b <= 7; ++b) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum[b] += __shfl_xor(sum[b], o);
    if (lane == 0) part[wave][b] = sum[b];
  }
  __syncthreads();
  if (t == 0) {
    unsigned long long tot[8] = {};
#pragma unroll
    for (uint32_t b = 1; b <= 7; ++b) tot[b] = part[0][b] + part[1][b] + part[2][b] + part[3][b];
    sc.gb[g] = pick_b(tot);
  }
}

// Validates a staged record header against the format for a block of m
// elements and the record length len.  Thread 0 only.
__device__ bool check_record_header(const Smem& s, uint32_t m, uint32_t len, uint32_t* mode, uint32_t* b,
                                    uint32_t* n_esc) {
  const uint4 r = s.stage[0];
  const uint32_t md = r.x & 0xFFu, bb = (r.x >> 8) & 0xFFu, reserved = r.x >> 16, rm = r.y, ne = r.z, rb = r.w;
  const bool ok = reserved == 0 && rm == m && rb == len &&
                  ((md == 0 && bb == 0 && ne == 0 && rb == raw_bytes(m)) ||
                   (md == 1 && m == kB && bb >= 1 && bb <= 7 && ne <= kB && rb == coded_bytes(bb, ne)));
  *mode = md; *b = bb; *n_esc = ne;
  return ok;
}

__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kCW))) void decompress_kernel(
    const uint8_t* __restrict__ in, uint64_t in_bytes, uint16_t* __restrict__ out, uint64_t n,
    int32_t* __restrict__ status, uint32_t nb) {
  __shared__ Smem s;
  const int t = threadIdx.x;
  const uint32_t bid = blockIdx.x;
  const uint64_t first = (uint64_t)bid * kB;
  const uint32_t m = (uint32_t)((n - first) < kB ? (n - first) : kB);
  if (t == 0) {
    uint64_t off = 0;
    uint32_t len = 0;
    s.plan[0] = check_stream(in, in_bytes, kMagic, n, nb, bid, &off, &len);
    s.plan[4] = len;
    s.misc[0] = off;
  }
  __syncthreads();
  if (!s.plan[0]) {
    if (t == 0) atomicExch(status, (int32_t)HC_ERR_CORRUPT_STREAM);
    return;
  }
  const uint32_t len = s.plan[4];
  copy_in(s, in + s.misc[0], len);  // the whole record, its header included
  __syncthreads();
  if (t == 0) {
    uint32_t mode = 0, b = 0, n_esc = 0;
    s.plan[0] = check_record_header(s, m, len, &mode, &b, &n_esc);
    s.plan[1] = mode; s.plan[2] = b; s.plan[3] = n_esc;
  }
  __syncthreads();
  if (!s.plan[0]) {
    if (t == 0) atomicExch(status, (int32_t)HC_ERR_CORRUPT_STREAM);
    return;
  }
  uint4 v[kPer];
  const bool ok = read_block(s, s.plan[1], s.plan[2], m, s.plan[3], len, v);
  if (!ok) {
    if (t == 0) atomicExch(status, (int32_t)HC_ERR_CORRUPT_STREAM);
    return;
  }
  store_block(out + first, m, v);
}

// After decoding: a corrupt stream leaves the whole output zero.
__global__ void zero_if_corrupt_kernel(const int32_t* status, uint32_t* out, size_t words, uint16_t* tail,
                                       int has_tail) {
  if (*status == 0) return;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    out[i] = 0;
  if (has_tail && blockIdx.x == 0 && threadIdx.x == 0) *tail = 0;
}

// ---------------------------------------------------------------------------
// compressed ring allreduce
// ---------------------------------------------------------------------------

// Reduce-scatter step 0: every rank compresses the slice it sends first.
__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kCW))) void car_first_kernel(RingPtrs ptr, CarGeom g) {
  __shared__ Smem s;
  const uint32_t p = blockIdx.x / g.nbs, blk = blockIdx.x % g.nbs;
  const uint32_t j = (p + g.R - 1) % g.R;  // sender p sends slice p-1
  const uint32_t m = block_elems(g, j, blk);
  if (m == 0) return;
  uint4 v[kPer];
  load_block(ptr.send[p] + (uint64_t)j * g.L + (uint64_t)blk * kB, m, v);
  const Plan pl = plan_block(v, m, s);
  write_block(v, pl, s);
  copy_out(s, slot(g, p, 0, blk), pl.rec_bytes);
  count_wire(g, pl.rec_bytes);
}

// Reduce-scatter step s: receiver q decompresses what q-1 sent, folds in its
// own slice, writes the result if this is the last step, and compresses it
// for the next hop.
__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kCW))) void car_rs_kernel(RingPtrs ptr, CarGeom g, uint32_t step) {
  __shared__ Smem s;
  const uint32_t q = blockIdx.x / g.nbs, blk = blockIdx.x % g.nbs;
  const uint32_t p = (q + g.R - 1) % g.R;
  const uint32_t j = (q + 2 * g.R - 2 - step) % g.R;
  const uint32_t m = block_elems(g, j, blk);
  if (m == 0) return;
  const uint64_t e0 = (uint64_t)j * g.L + (uint64_t)blk * kB;
  uint4 v[kPer];
  read_slot(s, slot(g, p, step & 1, blk), m, v);
  // The receiver's own data goes through the staging buffer, which the decode
  // has finished with: it costs no registers while the decoded block is live
  // (loaded into registers during the decode instead, it spills).
  load_block_lds(ptr.send[q] + e0, m, s);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    v[k] = hop_bf16x8(v[k], s.stage[ctid() + kCT * k]);
    // Pin each packed word: left alone, the compiler carries the two unpacked
    // halves of every sum into the encoder and runs out of registers there.
    asm volatile("" : "+v"(v[k].x), "+v"(v[k].y), "+v"(v[k].z), "+v"(v[k].w));
  }
  __syncthreads();  // the staging buffer is the histogram's next
  if (step == g.R - 2) store_block(ptr.recv[q] + e0, m, v);
  const Plan pl = plan_block(v, m, s);
  write_block(v, pl, s);
  copy_out(s, slot(g, q, (step + 1) & 1, blk), pl.rec_bytes);
  count_wire(g, pl.rec_bytes);
}

// All-gather step s: receiver q decompresses the finished slice from q-1 into
// its output and, unless this is the last step, forwards the same bytes.
__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kCW))) void car_ag_kernel(RingPtrs ptr, CarGeom g, uint32_t step,
                                                          uint32_t buf_in) {
  __shared__ Smem s;
  const uint32_t q = blockIdx.x / g.nbs, blk = blockIdx.x % g.nbs;
  const uint32_t p = (q + g.R - 1) % g.R;
  const uint32_t j = (q + 2 * g.R - 1 - step) % g.R;
  const uint32_t m = block_elems(g, j, blk);
  if (m == 0) return;
  const uint64_t e0 = (uint64_t)j * g.L + (uint64_t)blk * kB;
  uint4 v[kPer];
  read_slot(s, slot(g, p, buf_in, blk), m, v);
  store_block(ptr.recv[q] + e0, m, v);
  if (step + 2 < g.R) {
    const uint32_t rb = s.plan[4];
    copy_out(s, slot(g, q, buf_in ^ 1u, blk), rb);
    count_wire(g, rb);
  }
}

}  // namespace

hipError_t launch_fill_u32(void* dst, uint32_t value, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  size_t grid = (words + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((uint32_t)grid), dim3(256), 0, stream,
                     static_cast<uint32_t*>(dst), value, words);
  return hipGetLastError();
}

size_t compress_ws_bytes(size_t n) { return kCompressWsHeader + 8 * ceil_div(n, kB); }

uint32_t lookback_spin_limit() {
  const char* e = getenv("HC_LOOKBACK_SPIN_LIMIT");
  if (!e || !*e) return kSpinLimit;
  char* end = nullptr;
  const unsigned long v = strtoul(e, &end, 10);
  return (*end == 0 && v >= 1 && v <= 0xFFFFFFFFul) ? (uint32_t)v : kSpinLimit;
}

static_assert(kNoAllocScratchBytes >= kCompressWsHeader + 8 * (size_t)kNoAllocMaxBlocks,
              "the static scratch holds the look-back head and every block's descriptor");

hipError_t noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // this device's copy (it is current)
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_compress(const uint16_t* in, size_t n, void* out, uint64_t* out_bytes, void* ws,
                           hipStream_t stream) {
  const size_t nb = ceil_div(n, kB);
  if (nb == 0) {
    hipLaunchKernelGGL(empty_stream_kernel, dim3(1), dim3(1), 0, stream, static_cast<uint8_t*>(out), kMagic,
                       out_bytes);
    return hipGetLastError();
  }
  if (nb >= (1ull << 31)) return hipErrorInvalidValue;
  hipError_t e = launch_fill_u32(ws, 0u, compress_ws_bytes(n) / 4, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compress_kernel<false>, dim3((uint32_t)nb), dim3(kCT), 0, stream, in, (uint64_t)n,
                     static_cast<uint8_t*>(out), out_bytes, static_cast<CompressWs*>(ws), (uint32_t)nb, ScopeWs{},
                     1u, lookback_spin_limit());
  return hipGetLastError();
}

// Workspace of the three-round baseline: one slot per block, the sizes, the offsets.
size_t staged_ws_bytes(size_t n) {
  const size_t nb = ceil_div(n, kB);
  return align256(nb * kRawFull) + align256(4 * nb) + align256(8 * (nb + 1));
}

hipError_t launch_compress_staged(const uint16_t* in, size_t n, void* out, uint64_t* out_bytes, void* ws,
                                  hipStream_t stream) {
  const size_t nb = ceil_div(n, kB);
  if (nb == 0) return launch_empty_stream(out, kMagic, out_bytes, stream);
  if (nb >= (1ull << 31)) return hipErrorInvalidValue;
  uint8_t* slots = static_cast<uint8_t*>(ws);
  uint32_t* sizes = reinterpret_cast<uint32_t*>(slots + align256(nb * kRawFull));
  uint64_t* offs = reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(sizes) + align256(4 * nb));
  hipLaunchKernelGGL(staged_encode_kernel, dim3((uint32_t)nb), dim3(kCT), 0, stream, in, (uint64_t)n, slots, sizes);
  hipLaunchKernelGGL(staged_scan_kernel, dim3(1), dim3(1024), 0, stream, sizes, (uint32_t)nb, offs);
  hipLaunchKernelGGL(staged_copy_kernel, dim3((uint32_t)nb), dim3(256), 0, stream, slots, sizes, offs,
                     static_cast<uint8_t*>(out), (uint64_t)n, (uint32_t)nb, out_bytes);
  return hipGetLastError();
}

size_t compress_scoped_ws_bytes(size_t n) {
  const size_t full = n / kB;
  size_t off[5];
  return scope_layout(compress_ws_bytes(n), full, full, off);
}

hipError_t launch_compress_scoped(const uint16_t* in, size_t n, void* out, uint64_t* out_bytes, void* ws,
                                  size_t group, hipStream_t stream) {
  const size_t nb = ceil_div(n, kB), full = n / kB;
  if (nb == 0) return launch_compress(in, n, out, out_bytes, ws, stream);
  if (nb >= (1ull << 31)) return hipErrorInvalidValue;
  // groups larger than the stream are one group; this keeps G within 32 bits
  const size_t G = (group == 0 || group > full) ? (full ? full : 1) : group;
  const size_t groups = full ? ceil_div(full, G) : 0;
  size_t off[5];
  const size_t base = compress_ws_bytes(n);
  scope_layout(base, groups, full, off);
  char* w = static_cast<char*>(ws);
  ScopeWs sc{reinterpret_cast<uint32_t*>(w + off[0]), reinterpret_cast<uint16_t*>(w + off[1]),
             reinterpret_cast<uint8_t*>(w + off[2]), reinterpret_cast<uint32_t*>(w + off[3]),
             reinterpret_cast<uint32_t*>(w + off[4])};
  // zero the look-back head and descriptors, and the group histograms
  hipError_t e = launch_fill_u32(ws, 0u, base / 4, stream);
  if (e == hipSuccess && groups) e = launch_fill_u32(w + off[0], 0u, groups * 256, stream);
  if (e != hipSuccess) return e;
  if (full) {
    const uint32_t F = (uint32_t)full, Gu = (uint32_t)G;
    size_t chunk = kSumChunk;
    while (ceil_div(G, chunk) > 32768) chunk *= 2;   // keeps grid.y small
    const uint32_t chunks = (uint32_t)ceil_div(G, chunk);
    hipLaunchKernelGGL(scope_hist_kernel, dim3(F), dim3(kCT), 0, stream, in, sc, F);
    hipLaunchKernelGGL(scope_sum_kernel, dim3((uint32_t)groups, chunks), dim3(256), 0, stream, sc, Gu, F,
                       (uint32_t)chunk);
    hipLaunchKernelGGL(scope_rank_kernel, dim3((uint32_t)groups), dim3(256), 0, stream, sc);
    hipLaunchKernelGGL(scope_esc_kernel, dim3(F), dim3(128), 0, stream, sc, Gu);
    if (G <= 64)
      hipLaunchKernelGGL(scope_pick_small_kernel, dim3((uint32_t)ceil_div(groups, 256)), dim3(256), 0, stream, sc,
                         Gu, F, (uint32_t)groups);
    else
      hipLaunchKernelGGL(scope_pick_kernel, dim3((uint32_t)groups), dim3(256), 0, stream, sc, Gu, F);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(compress_kernel<true>, dim3((uint32_t)nb), dim3(kCT), 0, stream, in, (uint64_t)n,
                     static_cast<uint8_t*>(out), out_bytes, static_cast<CompressWs*>(ws), (uint32_t)nb, sc,
                     (uint32_t)G, lookback_spin_limit());
  return hipGetLastError();
}

hipError_t launch_empty_stream(void* out, uint32_t magic, uint64_t* out_bytes, hipStream_t stream) {
  hipLaunchKernelGGL(empty_stream_kernel, dim3(1), dim3(1), 0, stream, static_cast<uint8_t*>(out), magic, out_bytes);
  return hipGetLastError();
}

hipError_t launch_check_empty_stream(const void* in, size_t in_bytes, uint32_t magic, int32_t* status,
                                     hipStream_t stream) {
  hipLaunchKernelGGL(check_empty_stream_kernel, dim3(1), dim3(1), 0, stream, static_cast<const uint8_t*>(in),
                     (uint64_t)in_bytes, magic, status);
  return hipGetLastError();
}

hipError_t launch_decompress(const void* in, size_t in_bytes, uint16_t* out, size_t n, int32_t* status,
                             hipStream_t stream) {
  hipError_t e = launch_fill_u32(status, 0u, 1, stream);
  if (e != hipSuccess) return e;
  const size_t nb = ceil_div(n, kB);
  if (nb >= (1ull << 31)) return hipErrorInvalidValue;
  if (nb == 0) return launch_check_empty_stream(in, in_bytes, kMagic, status, stream);
  hipLaunchKernelGGL(decompress_kernel, dim3((uint32_t)nb), dim3(kCT), 0, stream,
                     static_cast<const uint8_t*>(in), (uint64_t)in_bytes, out, (uint64_t)n, status, (uint32_t)nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_zero_if_corrupt(status, out, n, stream);
}

hipError_t launch_zero_if_corrupt(const int32_t* status, uint16_t* out, size_t n, hipStream_t stream) {
  // A small grid: on a valid stream (the common case) every workgroup only
  // reads the status word and leaves; 64 workgroups still zero a corrupt
  // stream's output at a good fraction of the HBM rate.
  const size_t words = n / 2;
  size_t grid = (words + 255) / 256;
  if (grid > 64) grid = 64;
  if (grid == 0) grid = 1;
  hipLaunchKernelGGL(zero_if_corrupt_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, status,
                     reinterpret_cast<uint32_t*>(out), words, out + n - 1, (int)(n & 1));
  return hipGetLastError();
}

size_t compressed_ar_ws_bytes(size_t count, int R) {
  if (R < 1) return 0;
  const size_t L = ceil_div(count, (size_t)R);
  const size_t nbs = ceil_div(L, kB);
  return (size_t)R * 2 * nbs * kRawFull + 16;
}

hipError_t launch_compressed_allreduce(void* const* send, void* const* recv, size_t count, int R, size_t chunk,
                                       void* ws, uint64_t* wire_bytes, bool one_launch, Tap& tap,
                                       hipStream_t stream) {
  auto mark = [&]() -> hipError_t { return tap.mark(stream); };
  if (count == 0) {
    if (wire_bytes) hipLaunchKernelGGL(set_u64_kernel, dim3(1), dim3(1), 0, stream, wire_bytes, (uint64_t)0);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark();
    return e == hipSuccess ? tap.finish(stream) : e;   // every step empty
  }
  const size_t L = ceil_div(count, (size_t)R);
  const size_t nbs = ceil_div(L, kB);
  // Per (hop, chunk) stream framing bytes: the 32-byte header and the
  // offset table of every stream that crosses a link.  Records are added on
  // the device as they are produced.
  uint64_t framing = 0;
  for (int j = 0; j < R; ++j) {
    size_t lo = (size_t)j * L, hi = lo + L;
    if (lo > count) lo = count;
    if (hi > count) hi = count;
    for (size_t c0 = lo; c0 < hi; c0 += chunk) {
      const size_t len = (hi - c0) < chunk ? (hi - c0) : chunk;
      framing += 32 + round_up(8 * ceil_div(len, kB), 16);
    }
  }
  framing *= (uint64_t)2 * (R - 1);  // every slice crosses R-1 links in each phase
  if (wire_bytes) {
    hipLaunchKernelGGL(set_u64_kernel, dim3(1), dim3(1), 0, stream, wire_bytes, R > 1 ? framing : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (R == 1) {
    hipError_t e = mark();
    if (e == hipSuccess && send[0] != recv[0]) {
      Seg seg{send[0], nullptr, recv[0], count};
      e = launch_copy_step(&seg, 1, 2, 0, stream);
    }
    if (e == hipSuccess) e = mark();
    return e;
  }
  if ((uint64_t)R * nbs >= (1ull << 31)) return hipErrorInvalidValue;
  RingPtrs ptr;
  for (int r = 0; r < R; ++r) {
    ptr.send[r] = static_cast<const uint16_t*>(send[r]);
    ptr.recv[r] = static_cast<uint16_t*>(recv[r]);
  }
  CarGeom g;
  g.count = count;
  g.L = L;
  g.R = (uint32_t)R;
  g.nbs = (uint32_t)nbs;
  g.wire = static_cast<uint8_t*>(ws);
  g.wire_bytes = wire_bytes;
  const dim3 grid((uint32_t)(R * nbs)), block(kCT);
  if (!tap.ev && one_launch)   // no per-step timing asked for: one launch, each block through every hop
    return launch_car_chain(ptr, g, stream);
  hipError_t e = mark();
  if (e != hipSuccess) return e;
  void* first_args[] = {&ptr, &g};
  if ((e = launch_kernel((const void*)car_first_kernel, grid, block, first_args, stream)) != hipSuccess) return e;
  uint32_t step = 0, buf = 0;
  void* rs_args[] = {&ptr, &g, &step};
  for (int s = 0; s + 1 < R; ++s) {
    if ((e = mark()) != hipSuccess) return e;
    step = (uint32_t)s;   // the launch copies the argument values
    if ((e = launch_kernel((const void*)car_rs_kernel, grid, block, rs_args, stream)) != hipSuccess) return e;
  }
  // After reduce-scatter step R-2 the finished slice's record is in buffer (R-1)&1.
  buf = (uint32_t)((R - 1) & 1);
  void* ag_args[] = {&ptr, &g, &step, &buf};
  for (int s = 0; s + 1 < R; ++s) {
    if ((e = mark()) != hipSuccess) return e;
    step = (uint32_t)s;
    if ((e = launch_kernel((const void*)car_ag_kernel, grid, block, ag_args, stream)) != hipSuccess) return e;
    buf ^= 1u;
  }
  return mark();
}

}  // namespace hc
