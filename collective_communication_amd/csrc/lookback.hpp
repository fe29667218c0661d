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
// unpublished descriptor spin_limit times gives up, publishes poison (walks
// that reach it give up too), sets the error word and writes no record; the
// call then reports no stream (its byte count is 0) instead of hanging.  An earlier design took an atomic ticket per block to make the
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
constexpr uint64_t kFlagPoison = 3ull << 62;  // the block gave up: no valid prefix through it
constexpr uint64_t kValueMask = (1ull << 62) - 1;
constexpr uint32_t kSpinLimit = 1u << 22;   // polls of an unpublished descriptor before a walk gives up

// Workspace of a stream encoder: counts of ended walks, then one 64-bit
// look-back descriptor per block (all zero before the launch).
// Ended walks are counted in kWalkCounters counters, one per 128-byte line
// (block j adds to counter j % kWalkCounters): thousands of blocks adding to
// one address would queue behind each other at the memory side.
constexpr uint32_t kWalkCounters = 64;
struct CompressWs {
  uint32_t pad[32];
  uint64_t walked[kWalkCounters][16];   // word 0 of each line: blocks j % 64 == line whose walk ended,
                                        // in the low half; those that gave up, in the high half
  uint64_t desc[1];
};
constexpr size_t kCompressWsHeader = 128 + 128 * kWalkCounters;

__device__ __forceinline__ void publish(uint64_t* d, uint64_t v) {
  __hip_atomic_store(d, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t peek(uint64_t* d) {
  return __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One look-back window: lane l reads the descriptor of block base-l (blocks
// before 0 read as an inclusive prefix of 0).
__device__ __forceinline__ uint64_t lookback_peek(CompressWs* ws, int64_t base) {
  const int64_t j = base - (int64_t)__lane_id();
  return j >= 0 ? peek(&ws->desc[j]) : kFlagIncl;
}

// Byte offset of block bid's record among the records (the sum of the sizes
// of blocks 0..bid-1).  Called by the 64 lanes of one wave after the block
// published its own size.  Lane l reads the descriptor of block bid-1-l; the
// nearest predecessor with an inclusive prefix ends the walk and the sizes of
// the blocks between add to it; a window with an unpublished descriptor
// before that point is read again, a bounded number of times.
// Publishes the block's inclusive prefix and returns the exclusive one to
// every lane, with *ok true.  When a wait runs past its bound, or the walk
// ends at a poisoned predecessor, the block publishes poison instead (later
// walks that reach it give up too) and *ok is false: the caller then writes
// no record.  Either way the block then counts its ended walk
// (lookback_count_done).
__device__ __forceinline__ uint64_t lookback_wave(CompressWs* ws, uint32_t bid, uint32_t rec_bytes, uint32_t spin_limit,
                                                  bool* ok) {
  const uint32_t lane = __lane_id();
  uint64_t excl = 0;
  int64_t base = (int64_t)bid - 1;
  uint64_t d = lookback_peek(ws, base);
  uint32_t spins = 0;
  bool good = true;
  while (base >= 0) {
    const uint64_t end_mask = __ballot((d >> 62) >= 2);   // an inclusive prefix or poison
    const uint64_t zero_mask = __ballot((d >> 62) == 0);
    const int first = end_mask ? __ffsll((unsigned long long)end_mask) - 1 : 64;
    const uint64_t need = first == 64 ? ~0ull : ((2ull << first) - 1ull);
    if (zero_mask & need) {
      if (++spins >= spin_limit) {  // a predecessor never published: give up
        good = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      d = lookback_peek(ws, base);
      continue;
    }
    uint32_t agg = (int)lane < first ? (uint32_t)(d & kValueMask) : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) agg += __shfl_xor(agg, o, 64);
    excl += agg;
    if (first < 64) {
      const uint64_t e = lane_read64(d, (uint32_t)first);
      good = (e >> 62) == 2;
      excl += e & kValueMask;
      break;
    }
    base -= 64;
    d = lookback_peek(ws, base);
  }
  if (lane == 0 && bid != 0) publish(&ws->desc[bid], good ? (kFlagIncl | (excl + rec_bytes)) : kFlagPoison);
  *ok = good;
  return excl;
}

// Every block but the last counts its ended walk, and whether it gave up,
// in one 64-bit add: the count and the failure travel together, so no
// ordering between two locations (and no fence) is needed.
__device__ __forceinline__ void lookback_count_done(CompressWs* ws, uint32_t bid, bool ok) {
  __hip_atomic_fetch_add(&ws->walked[bid % kWalkCounters][0], ok ? 1ull : (1ull | (1ull << 32)), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

// The last block, after its own walk, with the 64 lanes of one wave: waits
// (bounded) until the other nb-1 blocks have counted their walks, then
// reports whether any gave up.  A walk that gave up at any time is therefore
// seen, even one the last block's own walk never reached (it summed that
// block's size instead).  True (in every lane) when the stream is not valid.
__device__ __forceinline__ bool lookback_failed(CompressWs* ws, uint32_t nb, uint32_t spin_limit) {
  static_assert(kWalkCounters == 64, "one counter per lane");
  const uint32_t lane = __lane_id();
  uint32_t spins = 0;
  for (;;) {
    const uint64_t w = __hip_atomic_load(&ws->walked[lane][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t done = (uint32_t)w, failed = (uint32_t)(w >> 32);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      done += __shfl_xor(done, o, 64);
      failed |= __shfl_xor(failed, o, 64);
    }
    if (done >= nb - 1) return failed != 0;
    if (++spins >= spin_limit) return true;
    __builtin_amdgcn_s_sleep(1);
  }
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
