// lookback.hpp -- the single-pass stream writer shared by the codecs.
//
// Block j of the stream is workgroup j.  Each block publishes the size of its
// record as soon as it knows it, then finds the record's byte offset by a
// decoupled look-back over the descriptors of the blocks before it, and
// writes the record straight into the final stream ("CCCL: In-GPU
// Compression-Coupled Collective Communication", section 4.4: one write
// round, no coalescing pass).
//
// Why the waits end.  A block waits only on lower-indexed blocks.  The
// dispatcher of each XCD starts the workgroups it is given in increasing
// index order.  So every workgroup that holds a slot on the XCD of the
// lowest-indexed unfinished workgroup has a lower index, has therefore
// finished, and has left a slot free: that workgroup starts, waits on
// nothing unfinished, and finishes; by induction all do.  That order is how
// the hardware dispatches, not a promise of the programming model, so every
// wait is also bounded: a walk that polls an
// unpublished descriptor kSpinLimit times sets the error word and gives up,
// and the call then reports no stream (its byte count is 0) instead of
// hanging.  An earlier design took an atomic ticket per block to make the
// order explicit; its round trip before each block's first load cost 23 us of
// a 269 us call on 2^28 elements, and no walk has timed out without it.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "codec.hpp"
#include "common.hpp"

namespace hc {

constexpr uint64_t kFlagAgg = 1ull << 62;     // descriptor holds the block's own size
constexpr uint64_t kFlagIncl = 2ull << 62;    // descriptor holds the size of blocks 0..bid
constexpr uint64_t kValueMask = (1ull << 62) - 1;
constexpr uint32_t kSpinLimit = 1u << 22;

// Workspace of a stream encoder: a spare word, an error word, then one
// 64-bit look-back descriptor per block (all zero before the launch).
struct CompressWs {
  uint32_t spare;
  uint32_t error;
  uint32_t pad[14];
  uint64_t desc[1];
};
constexpr size_t kCompressWsHeader = 64;

__device__ __forceinline__ void publish(uint64_t* d, uint64_t v) {
  __hip_atomic_store(d, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t peek(uint64_t* d) {
  return __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Byte offset of block bid's record among the records (the sum of the sizes
// of blocks 0..bid-1).  Called by the 64 lanes of one wave after the block
// published its own size; publishes the block's inclusive prefix and returns
// the exclusive one to every lane.  Lane l reads the descriptor of block
// bid-1-l; the nearest predecessor with an inclusive prefix ends the walk and
// the sizes of the blocks between add to it.  A window with an unpublished
// descriptor before that point is read again, a bounded number of times;
// then the error word is set and the walk gives up.
__device__ __forceinline__ uint64_t lookback_wave(CompressWs* ws, uint32_t bid, uint32_t rec_bytes) {
  const uint32_t lane = __lane_id();
  uint64_t excl = 0;
  int64_t base = (int64_t)bid - 1;
  uint32_t spins = 0;
  while (base >= 0) {
    const int64_t j = base - (int64_t)lane;
    const uint64_t d = j >= 0 ? peek(&ws->desc[j]) : kFlagIncl;
    const uint64_t incl_mask = __ballot((d >> 62) == 2);
    const uint64_t zero_mask = __ballot((d >> 62) == 0);
    const int first = incl_mask ? __ffsll((unsigned long long)incl_mask) - 1 : 64;
    const uint64_t need = first == 64 ? ~0ull : ((2ull << first) - 1ull);
    if (zero_mask & need) {
      if (++spins >= kSpinLimit) {  // a predecessor never published: give up, flag it
        if (lane == 0) atomicExch(&ws->error, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    uint32_t agg = (int)lane < first ? (uint32_t)(d & kValueMask) : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) agg += __shfl_xor(agg, o, 64);
    excl += agg;
    if (first < 64) {
      excl += lane_read64(d, (uint32_t)first) & kValueMask;
      break;
    }
    base -= 64;
  }
  if (lane == 0 && bid != 0) publish(&ws->desc[bid], kFlagIncl | (excl + rec_bytes));
  return excl;
}

// Stream container shared by the codec formats: a 32-byte header {u32 magic,
// u32 block elements, u64 n, u32 blocks, u32 0, u64 total bytes}, then one
// u64 record offset per block, padded to 16 bytes.
__device__ __forceinline__ uint32_t header_bytes(uint32_t nb) { return 32u + ((8u * nb + 15u) & ~15u); }

__device__ __forceinline__ void write_stream_header(uint8_t* out, uint32_t magic, uint32_t block, uint64_t n,
                                                    uint32_t nb, uint64_t total) {
  uint32_t* h = reinterpret_cast<uint32_t*>(out);
  h[0] = magic;
  h[1] = block;
  *reinterpret_cast<uint64_t*>(out + 8) = n;
  h[4] = nb;
  h[5] = 0;
  *reinterpret_cast<uint64_t*>(out + 24) = total;
  if (nb & 1u) *reinterpret_cast<uint64_t*>(out + 32 + 8ull * nb) = 0;  // table padding
}

// Validates the stream header and the offsets of block bid; on success
// returns the record's offset and length (next offset minus this one).
// All loads are independent, one round trip; any number of lanes may call it.
__device__ __forceinline__ bool check_stream(const uint8_t* in, uint64_t in_bytes, uint32_t magic, uint64_t n,
                                             uint32_t nb, uint32_t bid, uint64_t* off_out, uint32_t* len_out) {
  const uint64_t hdr = header_bytes(nb);
  if (in_bytes < hdr) return false;
  const uint64_t* offs = reinterpret_cast<const uint64_t*>(in + 32);
  const uint4 h0 = ld16(in), h1 = ld16(in + 16);
  const uint64_t off = offs[bid];
  const uint64_t next_off = bid + 1 < nb ? offs[bid + 1] : 0;
  const uint64_t pad = (bid == 0 && (nb & 1u)) ? offs[nb] : 0;
  const uint64_t hn = ((uint64_t)h0.w << 32) | h0.z;
  const uint64_t total = ((uint64_t)h1.w << 32) | h1.z;
  const uint64_t next = bid + 1 < nb ? next_off : total;
  const bool ok = h0.x == magic && h0.y == codec::kB && hn == n && h1.x == nb && h1.y == 0 && total <= in_bytes &&
                  total >= hdr && pad == 0 && (bid != 0 || off == hdr) && (off & 15u) == 0 && off >= hdr &&
                  next <= total && next >= off + 16 && next - off <= codec::kRawFull && ((next - off) & 15u) == 0;
  *off_out = off;
  *len_out = ok ? (uint32_t)(next - off) : 0u;
  return ok;
}

}  // namespace hc
