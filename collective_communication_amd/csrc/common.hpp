// common.hpp -- device helpers shared by the gfx950 kernels of libhc.
//
// Number rules (the hop of the ring, written for the GPU):
//  * fp32 hop: one IEEE binary32 add.  The library is built without fast-math
//    and with -ffp-contract=off, and gfx9 keeps fp32 subnormals by default.
//  * bf16 hop: widen both operands exactly (bf16 is the top half of an fp32
//    word), one fp32 add, round the sum to bf16 nearest-even.
//  * a NaN sum becomes the canonical quiet NaN (0x7FC00000 / 0x7FC0).
//  * SGD update (the fused allreduce + update): w - lr*g with the product and
//    the difference rounded once each in fp32 (no fused multiply-add); bf16
//    operands are widened exactly and the result rounded to bf16 as above.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

constexpr int kMaxRanks = 64;
constexpr int kThreads = 256;          // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t f32_bits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __uint_as_float(u); }

// Round an fp32 word to bf16, nearest even, by integer arithmetic: adding
// 0x7FFF plus the lowest kept bit carries into the kept half exactly when the
// dropped half is above the midpoint, or at it with an odd kept half.  A carry
// out of the largest finite value lands on the infinity encoding, which is
// IEEE overflow under round-to-nearest.
__device__ __forceinline__ uint32_t bf16_rne(uint32_t u) {
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}

__device__ __forceinline__ uint32_t hop_f32(uint32_t a, uint32_t b) {
  float s = bits_f32(a) + bits_f32(b);
  return (s != s) ? 0x7FC00000u : f32_bits(s);
}

// Two bf16 hops on a packed pair (low and high halves of a 32-bit word).
__device__ __forceinline__ uint32_t hop_bf16x2(uint32_t a, uint32_t b) {
  float lo = bits_f32(a << 16) + bits_f32(b << 16);
  float hi = bits_f32(a & 0xFFFF0000u) + bits_f32(b & 0xFFFF0000u);
  return bf16_rne(f32_bits(lo)) | (bf16_rne(f32_bits(hi)) << 16);
}

__device__ __forceinline__ uint4 hop_bf16x8(uint4 a, uint4 b) {
  return make_uint4(hop_bf16x2(a.x, b.x), hop_bf16x2(a.y, b.y), hop_bf16x2(a.z, b.z),
                    hop_bf16x2(a.w, b.w));
}

__device__ __forceinline__ uint4 hop_f32x4(uint4 a, uint4 b) {
  return make_uint4(hop_f32(a.x, b.x), hop_f32(a.y, b.y), hop_f32(a.z, b.z), hop_f32(a.w, b.w));
}

__device__ __forceinline__ uint32_t sgd_f32(uint32_t w, uint32_t g, float lr) {
  const float t = lr * bits_f32(g);
  const float r = bits_f32(w) - t;
  return (r != r) ? 0x7FC00000u : f32_bits(r);
}

// Two bf16 updates on packed pairs of weights and gradients.
__device__ __forceinline__ uint32_t sgd_bf16x2(uint32_t w, uint32_t g, float lr) {
  const float lo = bits_f32(w << 16) - lr * bits_f32(g << 16);
  const float hi = bits_f32(w & 0xFFFF0000u) - lr * bits_f32(g & 0xFFFF0000u);
  return bf16_rne(f32_bits(lo)) | (bf16_rne(f32_bits(hi)) << 16);
}

__device__ __forceinline__ uint4 sgd_bf16x8(uint4 w, uint4 g, float lr) {
  return make_uint4(sgd_bf16x2(w.x, g.x, lr), sgd_bf16x2(w.y, g.y, lr), sgd_bf16x2(w.z, g.z, lr),
                    sgd_bf16x2(w.w, g.w, lr));
}

__device__ __forceinline__ uint4 sgd_f32x4(uint4 w, uint4 g, float lr) {
  return make_uint4(sgd_f32(w.x, g.x, lr), sgd_f32(w.y, g.y, lr), sgd_f32(w.z, g.z, lr), sgd_f32(w.w, g.w, lr));
}

// Cross-lane reads.  The builtins return a signed int: widened into a 64-bit
// offset, a word with bit 31 set would sign-extend into a wild address.
// These return the 32-bit pattern unsigned; kernels read lanes only through
// them (a CPU lint over the sources keeps it so).
__device__ __forceinline__ uint32_t lane_read(uint32_t x, uint32_t lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, (int)lane);
}
__device__ __forceinline__ uint32_t first_lane_read(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ uint64_t lane_read64(uint64_t x, uint32_t lane) {
  return ((uint64_t)lane_read((uint32_t)(x >> 32), lane) << 32) | lane_read((uint32_t)x, lane);
}

// Streaming 16-byte global accesses.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

}  // namespace hc
