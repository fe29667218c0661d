// car.hpp -- device pieces of the fused compressed ring allreduce shared by
// its step-per-launch kernels (codec_kernels.hip) and its one-launch kernel
// (car_chain.hip): the rank pointers, the geometry of the wire slots, and the
// slot reader.  "CCCL: In-GPU Compression-Coupled Collective Communication",
// section 5 (selective compression) on the ring of "ResCCL: Resource-
// Efficient Scheduling for Collective Communication", section 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"
#include "launch.hpp"

namespace hc {
namespace codec {

// The same types in every file, whatever HC_CODEC_OPAQUE_TID is there.
struct RingPtrs {
  const uint16_t* send[kMaxRanks];
  uint16_t* recv[kMaxRanks];
};

struct CarGeom {
  uint64_t count;      // elements per rank buffer
  uint64_t L;          // slice length
  uint32_t R;
  uint32_t nbs;        // block slots per slice
  uint8_t* wire;       // R x 2 x nbs slots of kRawFull bytes
  uint64_t* wire_bytes;
};

// The one-launch schedule (car_chain.hip): every codec block of every slice
// through every hop, one workgroup each.
hipError_t launch_car_chain(const RingPtrs& ptr, const CarGeom& g, hipStream_t stream);

inline namespace HC_CODEC_TID_NS {

__device__ __forceinline__ uint8_t* slot(const CarGeom& g, uint32_t rank, uint32_t buf, uint32_t blk) {
  return g.wire + (((uint64_t)rank * 2 + buf) * g.nbs + blk) * kRawFull;
}

// Elements of block blk of slice j (0 when the block lies past the slice).
__device__ __forceinline__ uint32_t block_elems(const CarGeom& g, uint32_t j, uint32_t blk) {
  uint64_t lo = (uint64_t)j * g.L, hi = lo + g.L;
  if (lo > g.count) lo = g.count;
  if (hi > g.count) hi = g.count;
  const uint64_t b0 = lo + (uint64_t)blk * kB;
  if (b0 >= hi) return 0;
  return (uint32_t)((hi - b0) < kB ? (hi - b0) : kB);
}

__device__ __forceinline__ void count_wire(const CarGeom& g, uint32_t rec_bytes) {
  if (g.wire_bytes && ctid() == 0) atomicAdd((unsigned long long*)g.wire_bytes, (unsigned long long)rec_bytes);
}

// Reads a wire record produced by this library from a slot into LDS and
// decodes it.  The first kSpecVecs vectors of the slot are loaded with the
// record header, before its length is known (they lie inside the slot
// whatever the record is), so a record of up to kSpecVecs * 16 bytes takes
// one round trip.  The record header is clamped to the slot so that a
// damaged slot can never send a read out of bounds.
constexpr uint32_t kSpecPer = 3;                    // vectors per thread read ahead
constexpr uint32_t kSpecVecs = kSpecPer * kCT;      // 1536 vectors = 24 KB
static_assert(kSpecVecs <= kStage16, "read-ahead stays inside a slot");

__device__ __forceinline__ void read_slot(Smem& s, const uint8_t* src, uint32_t m, uint4 (&v)[kPer]) {
  const uint32_t t = ctid();
  uint4 pre[kSpecPer];
#pragma unroll
  for (uint32_t i = 0; i < kSpecPer; ++i) pre[i] = ld16(src + 16 * (t + kCT * i));
  if (t == 0) {
    const uint32_t mode = pre[0].x & 0xFFu, b = (pre[0].x >> 8) & 0xFFu, ne = pre[0].z, rb = pre[0].w;
    const bool ok = (mode == 0 && rb == raw_bytes(m)) ||
                    (mode == 1 && m == kB && b >= 1 && b <= 7 && ne <= kB && rb == coded_bytes(b, ne) &&
                     rb < kRawFull);
    s.plan[1] = ok ? mode : 0u;
    s.plan[2] = ok ? b : 0u;
    s.plan[3] = ok ? ne : 0u;
    s.plan[4] = ok ? rb : raw_bytes(m);
  }
  __syncthreads();
  const uint32_t mode = s.plan[1], b = s.plan[2], ne = s.plan[3], rb = s.plan[4];
  const uint32_t n16 = rb / 16u;
#pragma unroll
  for (uint32_t i = 0; i < kSpecPer; ++i)
    if (t + kCT * i < n16) s.stage[t + kCT * i] = pre[i];
  for (uint32_t i = kSpecVecs + t; i < n16; i += kCT) s.stage[i] = ld16(src + 16 * i);
  __syncthreads();
  read_block(s, mode, b, m, ne, rb, v);
}

}  // inline namespace HC_CODEC_TID_NS
}  // namespace codec
}  // namespace hc
