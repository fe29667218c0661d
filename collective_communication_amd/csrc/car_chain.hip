// car_chain.hip -- the fused compressed ring allreduce in one launch, for
// gfx950: workgroup (slice j, block b) compresses block b of slice j at its
// first sender and carries the record through every reduce-scatter and
// all-gather hop in ring order ("CCCL: In-GPU Compression-Coupled Collective
// Communication", section 5, on the ring of "ResCCL: Resource-Efficient
// Scheduling for Collective Communication", sections 1 and 3).
//
// Built with HC_CODEC_OPAQUE_TID: the codec helpers take their thread index
// through an opaque read, so the per-lane offsets of one hop are not held in
// registers across the loop over hops (they were hoisted out of it and
// spilled); this file holds only this kernel, and the one-block kernels keep
// the plain read.
#define HC_CODEC_OPAQUE_TID 1

#include "car.hpp"
#include "codec.hpp"
#include "launch.hpp"

namespace hc {
namespace codec {
namespace {

// One hop of a chain (see car_chain_kernel).  Reduce-scatter hop: fold the
// record in slot_in (none for the first hop) with the own block `own`, write
// the sum to `out` when given (the last step), compress it into slot_out.
__device__ __forceinline__ void chain_rs_hop(const uint8_t* slot_in, const uint16_t* own, uint16_t* out,
                                             uint8_t* slot_out, uint64_t* wire_bytes, uint32_t m, Smem& s) {
  slot_in = hop_ptr(slot_in);
  own = hop_ptr(own);
  out = hop_ptr(out);
  slot_out = hop_ptr(slot_out);
  wire_bytes = hop_ptr(wire_bytes);
  m = first_lane_read(m);
  uint4 v[kPer];
  if (!slot_in) {
    load_block(own, m, v);
  } else {
    read_slot(s, slot_in, m, v);
    load_block_lds(own, m, s);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      v[k] = hop_bf16x8(v[k], s.stage[ctid() + kCT * k]);
      asm volatile("" : "+v"(v[k].x), "+v"(v[k].y), "+v"(v[k].z), "+v"(v[k].w));
    }
    __syncthreads();
    if (out) store_block(out, m, v);
  }
  const Plan pl = plan_block(v, m, s);
  write_block(v, pl, s);
  copy_out(s, slot_out, pl.rec_bytes);
  if (wire_bytes && ctid() == 0) atomicAdd((unsigned long long*)wire_bytes, (unsigned long long)pl.rec_bytes);
  __syncthreads();   // the record is out of the staging buffer
}

// All-gather hop: decode the record in slot_in into `out`; forward the same
// bytes into slot_out when given.
__device__ __forceinline__ void chain_ag_hop(const uint8_t* slot_in, uint16_t* out, uint8_t* slot_out,
                                             uint64_t* wire_bytes, uint32_t m, Smem& s) {
  slot_in = hop_ptr(slot_in);
  out = hop_ptr(out);
  slot_out = hop_ptr(slot_out);
  wire_bytes = hop_ptr(wire_bytes);
  m = first_lane_read(m);
  uint4 v[kPer];
  read_slot(s, slot_in, m, v);
  store_block(out, m, v);
  if (slot_out) {
    const uint32_t rb = s.plan[4];
    copy_out(s, slot_out, rb);
    if (wire_bytes && ctid() == 0) atomicAdd((unsigned long long*)wire_bytes, (unsigned long long)rb);
  }
  __syncthreads();
}

// The whole compressed allreduce in one launch: workgroup (j, blk) carries
// codec block blk of slice j through every hop, in the ring's order, with
// the operations of the kernels above (the first sender compresses it; each
// reduce-scatter receiver decompresses, adds its own block, writes the sum at
// the last step and compresses again; each all-gather receiver decompresses
// into its output and forwards the same bytes).  A chunk's hops depend only
// on one another ("ResCCL: Resource-Efficient Scheduling for Collective
// Communication", section 3), so blocks never wait for each other; the slots
// are indexed by slice instead of by sending rank, since chains of different
// slices are at different hops at once (the same number of slots).  Same
// records, same wire bytes, same output as the step-per-launch schedule.
__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kCW))) void car_chain_kernel(RingPtrs ptr, CarGeom g) {
  __shared__ Smem s;
  const uint32_t j = blockIdx.x / g.nbs, blk = blockIdx.x % g.nbs;
  const uint32_t m = block_elems(g, j, blk);
  if (m == 0) return;
  const uint32_t R = g.R;
  const uint64_t e0 = (uint64_t)j * g.L + (uint64_t)blk * kB;
  for (uint32_t h = 0; h < R; ++h) {   // hop 0: the first sender j + 1; hop h: reduce-scatter step h - 1
    const uint32_t q = (j + 1 + h) % R;
    chain_rs_hop(h ? slot(g, j, (h - 1) & 1, blk) : nullptr, ptr.send[q] + e0,
                 h + 1 == R ? ptr.recv[q] + e0 : nullptr, slot(g, j, h & 1, blk), g.wire_bytes, m, s);
  }
  for (uint32_t step = 0; step + 1 < R; ++step) {   // all-gather step: receiver j + 1 + step
    const uint32_t q = (j + 1 + step) % R, buf = (R - 1 + step) & 1u;
    chain_ag_hop(slot(g, j, buf, blk), ptr.recv[q] + e0, step + 2 < R ? slot(g, j, buf ^ 1u, blk) : nullptr,
                 g.wire_bytes, m, s);
  }
}

}  // namespace

hipError_t launch_car_chain(const RingPtrs& ptr, const CarGeom& g, hipStream_t stream) {
  const dim3 grid(g.R * g.nbs), block(kCT);
  RingPtrs p = ptr;
  CarGeom gg = g;
  void* args[] = {&p, &gg};
  return launch_kernel((const void*)car_chain_kernel, grid, block, args, stream);
}

}  // namespace codec
}  // namespace hc
