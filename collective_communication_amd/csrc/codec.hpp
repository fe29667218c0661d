// codec.hpp -- one HCZ1 block (16384 bf16 = 32 KB) per 512-thread workgroup.
//
// The method is the exponent coder of "CCCL: In-GPU Compression-Coupled
// Collective Communication": section 4.1 (a bf16 word splits into sign,
// exponent and fraction; sign and fraction are sent as they are, the skewed
// 8-bit exponent is coded from a frequency table), section 4.3 (each block
// builds its own table; every symbol gets a fixed-length code) and section
// 4.4 (the block writes its output in one pass, no temporary buffers).  Byte
// format: see include/hc.h.
//
// gfx950 mapping.  Thread t of the workgroup owns the four 16-byte chunks
// c = t + 512k (k = 0..3) of the block, eight consecutive elements each, so
// every global load and store of a wave is a contiguous 1 KB.  Eight waves
// per block at no more than 64 VGPRs keep eight waves on every SIMD (LDS
// holds four blocks per CU): each wave's share of a block's serial latency
// chain is half what four waves of eight chunks would carry.  A chunk is
// exactly one byte of each code plane, which makes plane packing an 8x8
// bit-matrix transpose inside one register pair; the four lanes of a quad
// hold four consecutive chunks, so a byte transpose across the quad (two DPP
// moves and two v_perm_b32) turns their plane bytes into one 32-bit LDS
// store per plane.  The record is assembled in LDS (<= 32784 bytes) and
// leaves with 16-byte stores.
//   histogram : LDS atomics into 32 sub-histograms laid out bin-major
//               (lane l adds into copy l % 32, word 32e + copy, so the lanes
//               of a half-wave never share a bank and the address comes
//               straight out of the bf16 word with one AND-OR), held in the
//               staging buffer before the record needs it
//   ranking   : occurring exponents are compacted (ballot + popcount) into
//               a short list of keys (count desc, exponent asc) padded with
//               zero keys; eight lanes rank one key by counting the larger
//               ones, two 16-byte LDS reads per lane per 64 keys, and DPP
//               row shifts add their counts; absent exponents rank after
//               them in order
//   b choice  : a DPP prefix sum over the ranked counts gives the escape
//               count of every b; each wave reads the seven candidates with
//               readlane and keeps the smallest record (ties: smaller b)
//   escapes   : an element is an escape exactly when all b of its plane bits
//               are set, so the AND of the plane bytes is the escape mask;
//               a workgroup scan (DPP rows + one LDS exchange) orders them
//   decode    : for b <= 4 the dictionary sits in registers and v_perm_b32
//               maps four codes to four exponents at once
#pragma once

#include "common.hpp"

// HC_CODEC_OPAQUE_TID (0 unless the including file sets it first): the codec
// helpers read their thread index through an opaque read (see ctid below).
// Only a kernel that runs several blocks or hops in one loop wants it; the
// one-block kernels keep the plain read, whose values the compiler shares
// between helpers.  The two builds of the helpers live in differently named
// inline namespaces, so files built with different settings never share a
// definition.
#ifndef HC_CODEC_OPAQUE_TID
#define HC_CODEC_OPAQUE_TID 0
#endif
#if HC_CODEC_OPAQUE_TID
#define HC_CODEC_TID_NS opaque_tid
#else
#define HC_CODEC_TID_NS plain_tid
#endif

namespace hc {
namespace codec {
inline namespace HC_CODEC_TID_NS {

constexpr uint32_t kB = 16384;                  // elements per block
constexpr uint32_t kChunks = kB / 8;            // 16-byte chunks per block
constexpr int kCT = 512;                        // threads of a codec workgroup
constexpr int kCW = kCT / 64;                   // its waves
constexpr int kPer = kChunks / kCT;             // chunks per thread (4)
constexpr int kEmWords = (kPer + 3) / 4;        // words of packed per-chunk escape masks
static_assert(kPer % 2 == 0 && kPer <= 8 && kCT >= 256, "codec thread layout");
constexpr uint32_t kPlaneBytes = kB / 8;        // one code plane
constexpr uint32_t kRawFull = 16 + 2 * kB;      // raw record of a full block
constexpr uint32_t kStage16 = kRawFull / 16;    // 2049 uint4 of LDS staging
constexpr uint32_t kMagic = 0x315A4348u;
constexpr uint32_t kHistCopies = 32;            // 256 bins x 32 words = 32 KB of staging

// Thread and lane index of a codec thread (one-dimensional workgroups of kCT
// threads).  With HC_CODEC_OPAQUE_TID the index passes through an empty
// volatile asm, and every helper below takes it from a call of its own, so
// nothing the compiler derives from it (the per-lane LDS and global offsets)
// is shared between helper calls: a kernel that runs several hops in a loop
// then keeps no such value live across the loop, where it would be hoisted
// out and spilled.  Within one helper the values are shared as usual.
__device__ __forceinline__ uint32_t ctid() {
  uint32_t t = threadIdx.x;
#if HC_CODEC_OPAQUE_TID
  asm volatile("" : "+v"(t));
#endif
  return t;
}
__device__ __forceinline__ uint32_t clane() { return ctid() & 63u; }

// A global-memory pointer that every lane holds with the same value, read
// from the first lane (a convergent operation, which the compiler neither
// hoists out of a loop nor merges with another call) and rebuilt in the
// global address space.  A kernel that runs several hops in a loop passes its
// per-hop pointers through it, so that the per-lane addresses derived from
// them are formed inside each hop instead of being held across the loop.
template <class T>
__device__ __forceinline__ T* hop_ptr(T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint64_t u = ((uint64_t)first_lane_read((uint32_t)(a >> 32)) << 32) | first_lane_read((uint32_t)a);
  return (T*)(__attribute__((address_space(1))) T*)(uintptr_t)u;
}

struct Plan {
  uint32_t mode;       // 0 raw, 1 coded
  uint32_t b;          // code bits (coded)
  uint32_t K;          // dictionary entries = escape code
  uint32_t n_esc;
  uint32_t rec_bytes;
  uint32_t m;          // elements in the block
};

struct Smem {
  uint4 stage[kStage16 + 1];     // the record being built or read, plus a spare vector that
                                 // the decoder's 12-byte escape window may touch
  uint32_t key[256];             // (count << 8) | (255 - exponent) of occurring exponents
  uint32_t cbr[256];             // count by rank
  uint8_t code_of[256];          // exponent -> code
  uint8_t rank_of[256];          // exponent -> rank by (count desc, exponent asc)
  uint32_t wsum[kCW][4];         // per-wave totals (scans)
  uint32_t plan[8];
  uint64_t misc[2];
};

// The staging buffer of any workgroup's LDS struct with a `stage` member.
template <class S>
__device__ __forceinline__ uint8_t* stage8(S& s) { return reinterpret_cast<uint8_t*>(s.stage); }
template <class S>
__device__ __forceinline__ uint32_t* stage32(S& s) { return reinterpret_cast<uint32_t*>(s.stage); }

__host__ __device__ constexpr uint32_t dict_bytes(uint32_t b) { return (1u << b) < 16u ? 16u : (1u << b); }
__host__ __device__ constexpr uint32_t coded_bytes(uint32_t b, uint32_t n_esc) {
  return 16u + dict_bytes(b) + kPlaneBytes * b + kB + ((n_esc + 15u) & ~15u);
}
__host__ __device__ constexpr uint32_t raw_bytes(uint32_t m) { return 16u + ((2u * m + 15u) & ~15u); }
__host__ __device__ constexpr uint32_t planes_off(uint32_t b) { return 16u + dict_bytes(b); }
__host__ __device__ constexpr uint32_t sm_off(uint32_t b) { return planes_off(b) + kPlaneBytes * b; }
__host__ __device__ constexpr uint32_t esc_off(uint32_t b) { return sm_off(b) + kB; }

// ---------------------------------------------------------------------------
// cross-lane helpers
// ---------------------------------------------------------------------------

// DPP move: lanes whose source is outside the row read 0, rows outside
// ROW_MASK read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp0(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele steps
// inside each 16-lane row, then the row totals carried by row broadcasts.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp0<0x111>(x);          // row_shr:1
  x += dpp0<0x112>(x);          // row_shr:2
  x += dpp0<0x114>(x);          // row_shr:4
  x += dpp0<0x118>(x);          // row_shr:8
  x += dpp0<0x142, 0xA>(x);     // row_bcast:15 into rows 1 and 3
  x += dpp0<0x143, 0xC>(x);     // row_bcast:31 into rows 2 and 3
  return x;
}

// 4x4 byte transpose across the four lanes of a quad: lane i of the quad
// holds row i (bytes j = 0..3) and ends with column i.
__device__ __forceinline__ uint32_t quad_byte_transpose(uint32_t x, uint32_t lane) {
  const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  x = __builtin_amdgcn_perm(p1, x, (lane & 1u) ? 0x03070105u : 0x06020400u);
  const uint32_t p2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  return __builtin_amdgcn_perm(p2, x, (lane & 2u) ? 0x03020706u : 0x05040100u);
}

// 8x8 bit-matrix transpose of a 64-bit word held as (lo, hi): bit c of byte
// r moves to bit r of byte c.  Three rounds of delta swaps over 1x1, 2x2
// and 4x4 sub-blocks (the recursive block transpose of Hacker's Delight,
// section 7-3); the first two rounds stay inside each 32-bit half.  The
// transpose is its own inverse.
__device__ __forceinline__ void transpose8(uint32_t& lo, uint32_t& hi) {
  uint32_t t;
  t = (lo ^ (lo >> 7)) & 0x00AA00AAu; lo = lo ^ t ^ (t << 7);
  t = (hi ^ (hi >> 7)) & 0x00AA00AAu; hi = hi ^ t ^ (t << 7);
  t = (lo ^ (lo >> 14)) & 0x0000CCCCu; lo = lo ^ t ^ (t << 14);
  t = (hi ^ (hi >> 14)) & 0x0000CCCCu; hi = hi ^ t ^ (t << 14);
  t = (lo ^ (hi << 4)) & 0xF0F0F0F0u;
  lo ^= t;
  hi ^= t >> 4;
}

__device__ __forceinline__ uint32_t exp_lo(uint32_t w) { return (w >> 7) & 0xFFu; }
__device__ __forceinline__ uint32_t exp_hi(uint32_t w) { return (w >> 23) & 0xFFu; }

// Exponent bytes of four bf16 (two words), in element order.  Shifting a
// word left by one puts the exponent of its low element in byte 1 and that
// of its high element in byte 3.
__device__ __forceinline__ uint32_t exps4(uint32_t w0, uint32_t w1) {
  return __builtin_amdgcn_perm(w1 << 1, w0 << 1, 0x07050301u);
}

// Sign/fraction bytes of four bf16 (two words): byte = sign << 7 | fraction.
__device__ __forceinline__ uint32_t sm_quad(uint32_t w0, uint32_t w1) {
  const uint32_t lows = __builtin_amdgcn_perm(w1, w0, 0x06040200u);   // low byte of each element
  const uint32_t highs = __builtin_amdgcn_perm(w1, w0, 0x07050301u);  // high byte of each element
  return (lows & 0x7F7F7F7Fu) | (highs & 0x80808080u);
}

// Four bf16 rebuilt from their sign/fraction bytes S and exponent bytes E,
// as two words (elements 0,1 and 2,3).
__device__ __forceinline__ uint2 rebuild_quad(uint32_t S, uint32_t E) {
  const uint32_t H = (S & 0x80808080u) | ((E >> 1) & 0x7F7F7F7Fu);   // sign, exponent bits 7..1
  const uint32_t L = (S & 0x7F7F7F7Fu) | ((E << 7) & 0x80808080u);   // exponent bit 0, fraction
  return make_uint2(__builtin_amdgcn_perm(H, L, 0x05010400u), __builtin_amdgcn_perm(H, L, 0x07030602u));
}

__device__ __forceinline__ uint32_t chunk_elem_word(const uint4& v, int i) {
  const uint32_t w = (i < 2) ? v.x : (i < 4) ? v.y : (i < 6) ? v.z : v.w;
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}


// Escape masks of a thread's chunks, one byte each, packed four to a word:
// chunk k in byte k % 4 of word k / 4.
__device__ __forceinline__ uint32_t mask_of(const uint32_t (&em)[kEmWords], int k) {
  return (em[k >> 2] >> (8 * (k & 3))) & 0xFFu;
}

__device__ __forceinline__ uint32_t field16(const uint32_t* w, int k) {
  return (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
}

// Workgroup exclusive scan of the escape counts popc(mask k) (each <= 8) in
// element index order (chunk c = t + kCT * k, so k-major, then thread).
// Returns for each k the number of escapes before this thread's chunk k,
// and the total.  Counters travel as 16-bit fields, two per 32-bit word
// (a field never exceeds 8 * kCT).
__device__ __forceinline__ uint32_t block_excl_scan(const uint32_t (&em)[kEmWords], uint32_t (&excl)[kPer],
                                                    Smem& s) {
  constexpr int kW = kPer / 2;
  uint32_t mine[kW], incl[kW];
#pragma unroll
  for (int i = 0; i < kW; ++i) {
    mine[i] = __popc(mask_of(em, 2 * i)) | (__popc(mask_of(em, 2 * i + 1)) << 16);
    incl[i] = wave_incl_scan(mine[i]);
  }
  const int wave = ctid() >> 6;
  if (clane() == 63) {
#pragma unroll
    for (int i = 0; i < kW; ++i) s.wsum[wave][i] = incl[i];
  }
  __syncthreads();
  uint32_t before[kW], total[kW];
#pragma unroll
  for (int i = 0; i < kW; ++i) before[i] = total[i] = 0;
#pragma unroll
  for (int w = 0; w < kCW; ++w) {
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      const uint32_t x = s.wsum[w][i];
      before[i] += w < wave ? x : 0u;
      total[i] += x;
    }
  }
  uint32_t base = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    excl[k] = base + field16(before, k) + field16(incl, k) - field16(mine, k);
    base += field16(total, k);
  }
  return base;
}

// Loads a block's elements: thread t gets chunks t + 512k.  Elements at or
// past m read as zero.
__device__ __forceinline__ void load_block(const uint16_t* src, uint32_t m, uint4 (&v)[kPer]) {
  const int t = ctid();
  if (m == kB) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = ld16(src + 8 * (t + kCT * k));
    return;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t e0 = 8u * (t + kCT * k);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i)
      if (e0 + i < m) w[i >> 1] |= (uint32_t)src[e0 + i] << (16 * (i & 1));
    v[k] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Loads a block's elements into the staging buffer, chunk c at stage[c]: a
// full block with direct global->LDS 16-byte loads (each wave instruction
// fills 1 KB of LDS from 64 consecutive chunks and holds no registers), a
// partial one element by element with zeros past m.  Ends with a barrier.
__device__ __forceinline__ void load_block_lds(const uint16_t* src, uint32_t m, Smem& s) {
  const uint32_t t = ctid();
  if (m == kB) {
    const uint32_t lane = clane(), wave = t >> 6;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const uint32_t c0 = kCT * k + 64u * wave;  // first chunk of this wave's 1 KB
      __builtin_amdgcn_global_load_lds(src + 8 * (c0 + lane),
                                       (__attribute__((address_space(3))) void*)&s.stage[c0], 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // LDS DMA completes on the vector memory counter
  } else {
    uint4 one[1];
#pragma unroll 1
    for (int k = 0; k < kPer; ++k) {
      const uint32_t c = t + kCT * k;
      const uint32_t e0 = 8u * c;
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (uint32_t i = 0; i < 8; ++i)
        if (e0 + i < m) w[i >> 1] |= (uint32_t)src[e0 + i] << (16 * (i & 1));
      one[0] = make_uint4(w[0], w[1], w[2], w[3]);
      s.stage[c] = one[0];
    }
  }
  __syncthreads();
}

// Stores a block's elements (first m only).
__device__ __forceinline__ void store_block(uint16_t* dst, uint32_t m, const uint4 (&v)[kPer]) {
  const int t = ctid();
  if (m == kB) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) st16(dst + 8 * (t + kCT * k), v[k]);
    return;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t e0 = 8u * (t + kCT * k);
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i)
      if (e0 + i < m) dst[e0 + i] = (uint16_t)chunk_elem_word(v[k], (int)i);
  }
}

// ---------------------------------------------------------------------------
// encoding
// ---------------------------------------------------------------------------

// Phase 1 of encoding: histogram, ranking, the choice of b and the record
// size.  Leaves code_of[] and the dictionary in LDS; returns the plan
// (uniform).  Ends with a barrier.
// Clears the sub-histograms (the first 32 KB of the staging buffer).  The
// caller puts a barrier between this and plan_block<true>.
template <class S>
__device__ __forceinline__ void zero_hist(S& s) {
#pragma unroll
  for (int i = 0; i < (int)(kHistCopies * 256 / 4 / kCT); ++i) s.stage[ctid() + kCT * i] = make_uint4(0, 0, 0, 0);
}

// 256-bin histogram of a full block's exponents.  Returns the count of
// exponent t to thread t < 256 (the "owner" of bin t) and 0 to the others;
// the sub-histograms stay in the staging buffer.  ZEROED: the caller cleared
// them (zero_hist) and passed a barrier since.  Ends with no barrier after
// the owners' reads: the caller syncs before reusing the staging buffer.
//
// 32 sub-histograms, bin-major: the count of exponent e in copy c is word
// 32e + c.  Lane l adds into copy l % 32, so the 32 lanes of a half-wave
// always hit 32 different banks, and the byte address of bin e is e << 7 OR
// c << 2: for the low element of a word that is the word ANDed with 0x7F80
// (its exponent field already sits at bit 7).  Thread t sums the 32 copies
// of bin t: eight 16-byte reads, started at a different quad in each group of
// eight lanes to spread the banks.
template <bool ZEROED = false, class S>
__device__ __forceinline__ uint32_t block_histogram(const uint4 (&v)[kPer], S& s) {
  const uint32_t t = ctid(), lane = clane();
  uint8_t* sub8 = stage8(s);
  if constexpr (!ZEROED) {
    zero_hist(s);
    __syncthreads();
  }
  {
    const uint32_t c4 = (lane & (kHistCopies - 1)) << 2;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        atomicAdd(reinterpret_cast<uint32_t*>(sub8 + ((w4[q] & 0x7F80u) | c4)), 1u);
        atomicAdd(reinterpret_cast<uint32_t*>(sub8 + (((w4[q] >> 16) & 0x7F80u) | c4)), 1u);
      }
    }
  }
  __syncthreads();
  uint32_t cnt = 0;
  if (t < 256u) {
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i) {
      const uint4 q = s.stage[t * 8 + ((i + t) & 7u)];
      cnt += q.x + q.y + q.z + q.w;
    }
  }
  return cnt;
}

// ZEROED: the caller has already cleared the sub-histograms (zero_hist) and
// passed a barrier since.
template <bool ZEROED = false>
__device__ __forceinline__ Plan plan_block(const uint4 (&v)[kPer], uint32_t m, Smem& s) {
  const uint32_t t = ctid(), lane = clane();
  Plan p;
  p.m = m;
  if (m != kB) {  // partial blocks travel raw
    p.mode = 0; p.b = 0; p.K = 0; p.n_esc = 0; p.rec_bytes = raw_bytes(m);
    return p;
  }
  const bool owner = t < 256u;
  const uint32_t cnt = block_histogram<ZEROED>(v, s);
  // Rank = position in (count desc, exponent asc); key order is that order.
  const uint32_t key = (cnt << 8) | (255u - t);
  const uint64_t nzmask = __ballot(cnt > 0);
  const uint32_t wave = t >> 6;
  const uint32_t below = (uint32_t)__popcll(nzmask & ((1ull << lane) - 1ull));
  if (owner && lane == 0) s.wsum[wave][0] = (uint32_t)__popcll(nzmask);
  __syncthreads();
  uint32_t before = 0, nz_total = 0;
#pragma unroll
  for (uint32_t w = 0; w < 4u; ++w) {  // the owner waves
    const uint32_t c = s.wsum[w][0];
    before += w < wave ? c : 0;
    nz_total += c;
  }
  const uint32_t nz_below = before + below;
  // An exponent that never occurs ranks after all that do, in exponent order;
  // the occurring ones are compacted into a short list of keys, padded with
  // zero keys to a multiple of 64 (a zero key is below every real one).
  const uint32_t npad = (nz_total + 63u) & ~63u;
  if (owner) {
    if (cnt > 0) {
      s.key[nz_below] = key;
    } else {
      const uint32_t r = nz_total + (t - nz_below);
      s.cbr[r] = 0;
      s.rank_of[t] = (uint8_t)r;
    }
    if (t >= nz_total && t < npad) s.key[t] = 0;
  }
  __syncthreads();
  // rank(key i) = #{keys j > key i} (keys are distinct).  Eight lanes rank
  // one key: lane g of the group compares it with keys 8g .. 8g+7 of every
  // run of 64 (two 16-byte LDS reads, the same for all groups of a wave),
  // and three DPP row shifts add the eight partial counts into lane 7 of the
  // group.  64 keys per pass over the workgroup's 512 lanes; a wave whose
  // keys all lie past the list stops.
  for (uint32_t i0 = 0; i0 < nz_total; i0 += kCT / 8) {
    if (i0 + 8u * wave >= nz_total) break;  // wave-uniform
    const uint32_t i = i0 + (t >> 3), g = t & 7u;
    const uint32_t ki = i < nz_total ? s.key[i] : 0xFFFFFFFFu;
    uint32_t c = 0;
    for (uint32_t j0 = 0; j0 < npad; j0 += 64) {
      const uint4 a = *reinterpret_cast<const uint4*>(&s.key[j0 + 8u * g]);
      const uint4 b = *reinterpret_cast<const uint4*>(&s.key[j0 + 8u * g + 4u]);
      c += (uint32_t)(a.x > ki) + (uint32_t)(a.y > ki) + (uint32_t)(a.z > ki) + (uint32_t)(a.w > ki) +
           (uint32_t)(b.x > ki) + (uint32_t)(b.y > ki) + (uint32_t)(b.z > ki) + (uint32_t)(b.w > ki);
    }
    c += dpp0<0x111>(c);  // row_shr:1
    c += dpp0<0x112>(c);  // row_shr:2
    c += dpp0<0x114>(c);  // row_shr:4: lane 8m+7 holds the group's sum
    if (g == 7u && i < nz_total) {
      s.cbr[c] = ki >> 8;
      s.rank_of[255u - (ki & 0xFFu)] = (uint8_t)c;
    }
  }
  __syncthreads();
  // cover(K) = sum of the K largest counts, K = 2^b - 1.  Lane l holds ranks
  // 2l and 2l+1; after the inclusive scan S_l covers ranks <= 2l+1, and
  // cover(2^b - 1) = S_l - cbr[2l+1] at lane l = 2^(b-1) - 1.  Every wave
  // computes the same plan.
  {
    const uint32_t a = s.cbr[2 * lane], bb = s.cbr[2 * lane + 1];
    const uint32_t cover = wave_incl_scan(a + bb) - bb;
    uint32_t best = 0xFFFFFFFFu;
#pragma unroll
    for (uint32_t b = 1; b <= 7; ++b) {
      const uint32_t cov = lane_read(cover, (1u << (b - 1)) - 1u);
      const uint32_t size = coded_bytes(b, kB - cov);
      const uint32_t cand = (size << 3) | b;
      best = cand < best ? cand : best;
    }
    const uint32_t b = best & 7u, size = best >> 3;
    if (size < kRawFull) {
      p.mode = 1; p.b = b; p.K = (1u << b) - 1u;
      p.n_esc = kB - lane_read(cover, (1u << (b - 1)) - 1u);
      p.rec_bytes = size;
    } else {
      p.mode = 0; p.b = 0; p.K = 0; p.n_esc = 0; p.rec_bytes = kRawFull;
    }
  }
  if (p.mode == 1 && owner) {
    const uint32_t rank = s.rank_of[t];
    s.code_of[t] = (uint8_t)(rank < p.K ? rank : p.K);
    if (rank < dict_bytes(p.b)) stage8(s)[16 + rank] = rank < p.K ? (uint8_t)t : (uint8_t)0;
  }
  __syncthreads();
  return p;
}

// Shared code tables (the table-scope variant): the plan of a full block
// from its group's symbol order (rank -> exponent, 256 bytes), the group's
// code length b and the block's escape count for that b; a coded record is
// not smaller than the raw one travels raw.  Leaves code_of[] and the
// dictionary in LDS like plan_block.  Ends with a barrier.
__device__ __forceinline__ Plan given_plan(const uint8_t* order, uint32_t b, uint32_t n_esc, uint32_t m, Smem& s) {
  const uint32_t t = ctid();
  Plan p;
  p.m = m;
  p.mode = 0; p.b = 0; p.K = 0; p.n_esc = 0; p.rec_bytes = raw_bytes(m);
  if (m == kB && b >= 1 && b <= 7 && coded_bytes(b, n_esc) < kRawFull) {
    p.mode = 1; p.b = b; p.K = (1u << b) - 1u; p.n_esc = n_esc; p.rec_bytes = coded_bytes(b, n_esc);
  }
  if (p.mode == 1 && t < 256u) {
    const uint32_t sym = order[t];   // the exponent of rank t
    s.code_of[sym] = (uint8_t)(t < p.K ? t : p.K);
    if (t < dict_bytes(p.b)) stage8(s)[16 + t] = t < p.K ? (uint8_t)sym : (uint8_t)0;
  }
  __syncthreads();
  return p;
}

// Codes of four elements (two words), one byte each in element order.  The
// table bytes are loaded into 16-bit halves, two per register, and one byte
// permute packs the four.
__device__ __forceinline__ uint32_t codes4(const uint8_t* code_of, uint32_t w0, uint32_t w1) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  const us2 a = {code_of[exp_lo(w0)], code_of[exp_hi(w0)]};
  const us2 b = {code_of[exp_lo(w1)], code_of[exp_hi(w1)]};
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a), 0x06040200u);
}

// Writes the coded record of a block with B-bit codes into the staging
// buffer (everything after the 16-byte header and the dictionary).
template <int B>
__device__ __forceinline__ void write_coded(const uint4 (&v)[kPer], const Plan& p, Smem& s) {
  constexpr uint32_t poff = planes_off(B), soff = sm_off(B), eoff = esc_off(B);
  const uint32_t t = ctid(), lane = clane(), qi = lane & 3u;
  uint8_t* st = stage8(s);
  uint32_t* st32 = stage32(s);
  uint32_t escmask[kEmWords] = {};
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t c = t + kCT * k;
    const uint32_t w0 = v[k].x, w1 = v[k].y, w2 = v[k].z, w3 = v[k].w;
    uint32_t lo = codes4(s.code_of, w0, w1), hi = codes4(s.code_of, w2, w3);
    transpose8(lo, hi);  // now byte j of (lo, hi) = plane j of this chunk
    uint32_t em = lo;
#pragma unroll
    for (int j = 1; j < B; ++j) em &= (j < 4 ? lo >> (8 * j) : hi >> (8 * (j - 4)));
    em &= 0xFFu;
    const uint32_t col_lo = quad_byte_transpose(lo, lane);
    if (qi < (uint32_t)B) st32[(poff + qi * kPlaneBytes + (c - qi)) >> 2] = col_lo;
    if constexpr (B > 4) {
      const uint32_t col_hi = quad_byte_transpose(hi, lane);
      if (qi < (uint32_t)(B - 4)) st32[(poff + (4 + qi) * kPlaneBytes + (c - qi)) >> 2] = col_hi;
    }
    *reinterpret_cast<uint2*>(st + soff + 8 * c) = make_uint2(sm_quad(w0, w1), sm_quad(w2, w3));
    escmask[k >> 2] |= em << (8 * (k & 3));
  }
  if (p.n_esc) {
    uint32_t excl[kPer];
    block_excl_scan(escmask, excl, s);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      uint32_t em = mask_of(escmask, k), pos = excl[k];
      if (em) {
        const uint32_t e03 = exps4(v[k].x, v[k].y), e47 = exps4(v[k].z, v[k].w);
        while (em) {
          const uint32_t i = (uint32_t)__builtin_ctz(em);
          em &= em - 1;
          st[eoff + pos++] = (uint8_t)__builtin_amdgcn_perm(e47, e03, 0x0C0C0C00u | i);
        }
      }
    }
    const uint32_t pad_end = (p.n_esc + 15u) & ~15u;
    if (t < pad_end - p.n_esc) st[eoff + p.n_esc + t] = 0;
  }
}

// Phase 2 of encoding: writes the record for plan p into the LDS staging
// buffer.  Ends with a barrier.
__device__ __forceinline__ void write_block(const uint4 (&v)[kPer], const Plan& p, Smem& s) {
  const uint32_t t = ctid();
  if (t == 0) {
    uint32_t* h = stage32(s);
    h[0] = p.mode | (p.b << 8);
    h[1] = p.m;
    h[2] = p.n_esc;
    h[3] = p.rec_bytes;
  }
  if (p.mode == 0) {
    const uint32_t n16 = (p.rec_bytes - 16u) / 16u;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const uint32_t c = t + kCT * k;
      if (c < n16) s.stage[1 + c] = v[k];
    }
  } else {
    switch (p.b) {
      case 1: write_coded<1>(v, p, s); break;
      case 2: write_coded<2>(v, p, s); break;
      case 3: write_coded<3>(v, p, s); break;
      case 4: write_coded<4>(v, p, s); break;
      case 5: write_coded<5>(v, p, s); break;
      case 6: write_coded<6>(v, p, s); break;
      default: write_coded<7>(v, p, s); break;
    }
  }
  __syncthreads();
}

// Copies a staged record (rec_bytes, a multiple of 16) to global memory.
template <class S>
__device__ __forceinline__ void copy_out(const S& s, uint8_t* dst, uint32_t rec_bytes) {
  const uint32_t n16 = rec_bytes / 16u;
  for (uint32_t i = ctid(); i < n16; i += kCT) st16(dst + 16 * i, s.stage[i]);
}

// Copies a record from global memory into the staging buffer.
template <class S>
__device__ __forceinline__ void copy_in(S& s, const uint8_t* src, uint32_t rec_bytes) {
  const uint32_t n16 = rec_bytes / 16u;
  for (uint32_t i = ctid(); i < n16; i += kCT) s.stage[i] = ld16(src + 16 * i);
}

// ---------------------------------------------------------------------------
// decoding
// ---------------------------------------------------------------------------

// Exponents of four elements from their codes (one byte each, < 2^B); d holds
// the first 16 dictionary bytes.
template <int B>
__device__ __forceinline__ uint32_t lookup4(uint32_t codes, const uint32_t (&d)[4], const uint8_t* dict) {
  if constexpr (B <= 3) {
    return __builtin_amdgcn_perm(d[1], d[0], codes);
  } else if constexpr (B == 4) {
    const uint32_t c7 = codes & 0x07070707u;
    const uint32_t a = __builtin_amdgcn_perm(d[1], d[0], c7);
    const uint32_t b = __builtin_amdgcn_perm(d[3], d[2], c7);
    const uint32_t sel = ((codes >> 3) & 0x01010101u) * 0xFFu;
    return (b & sel) | (a & ~sel);
  } else {
    return (uint32_t)dict[codes & 0xFFu] | ((uint32_t)dict[(codes >> 8) & 0xFFu] << 8) |
           ((uint32_t)dict[(codes >> 16) & 0xFFu] << 16) | ((uint32_t)dict[codes >> 24] << 24);
  }
}

template <int B>
__device__ __forceinline__ bool read_coded(Smem& s, uint32_t n_esc, uint4 (&v)[kPer]) {
  constexpr uint32_t K = (1u << B) - 1u;
  constexpr uint32_t poff = planes_off(B), soff = sm_off(B), eoff = esc_off(B);
  const uint32_t t = ctid();
  const uint8_t* st = stage8(s);
  const uint32_t* st32 = stage32(s);
  bool bad = false;
  if (t >= K && t < dict_bytes(B)) bad |= st[16 + t] != 0;  // dictionary padding must be zero
  const uint32_t d[4] = {st32[4], st32[5], st32[6], st32[7]};
  uint32_t clo[kPer], chi[kPer], escmask[kEmWords] = {};
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t c = t + kCT * k;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const uint32_t byte = st[poff + j * kPlaneBytes + c];
      if (j < 4) lo |= byte << (8 * j);
      else hi |= byte << (8 * (j - 4));
    }
    uint32_t em = lo;
#pragma unroll
    for (int j = 1; j < B; ++j) em &= (j < 4 ? lo >> (8 * j) : hi >> (8 * (j - 4)));
    em &= 0xFFu;
    transpose8(lo, hi);  // now byte i of (lo, hi) = code of element i
    clo[k] = lo;
    chi[k] = hi;
    escmask[k >> 2] |= em << (8 * (k & 3));
  }
  uint32_t excl[kPer];
  const uint32_t total = block_excl_scan(escmask, excl, s);
  const bool count_ok = total == n_esc;
  const uint32_t pad_end = (n_esc + 15u) & ~15u;
  if (t < pad_end - n_esc) bad |= st[eoff + n_esc + t] != 0;  // escape padding must be zero
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t c = t + kCT * k;
    uint32_t E0 = lookup4<B>(clo[k], d, st + 16);
    uint32_t E1 = lookup4<B>(chi[k], d, st + 16);
    uint32_t em = mask_of(escmask, k);
    if (em && count_ok) {
      // Escaped elements take their exponents, in order, from the escape
      // plane bytes excl[k] .. excl[k] + popc - 1 (at most 8): three aligned
      // words cover them, and the lookup left a zero byte at every escaped
      // position (the dictionary entry of code K is zero padding).
      const uint32_t a = eoff + excl[k];  // + popc <= rec_bytes <= kRawFull: the spare vector covers the rest
      const uint32_t* w = st32 + (a >> 2);
      const uint32_t d0 = w[0], d1 = w[1], d2 = w[2];
      const uint32_t x0 = __builtin_amdgcn_alignbyte(d1, d0, a & 3u), x1 = __builtin_amdgcn_alignbyte(d2, d1, a & 3u);
      uint32_t j = 0;
      while (em) {
        const uint32_t i = (uint32_t)__builtin_ctz(em);
        em &= em - 1;
        const uint32_t e = __builtin_amdgcn_perm(x1, x0, 0x0C0C0C00u | j);
        ++j;
        if (i < 4) E0 |= e << (8u * i);
        else E1 |= e << (8u * (i - 4u));
      }
    }
    const uint2 smv = *reinterpret_cast<const uint2*>(st + soff + 8 * c);
    const uint2 a = rebuild_quad(smv.x, E0), b = rebuild_quad(smv.y, E1);
    v[k] = make_uint4(a.x, a.y, b.x, b.y);
  }
  return !__syncthreads_or(bad || !count_ok);
}

// Decodes the staged record (header already validated for mode, b, m,
// rec_bytes) into v.  Returns false (uniform) when the escape count or a
// padding byte disagrees with the format.  Ends with a barrier.
__device__ __forceinline__ bool read_block(Smem& s, uint32_t mode, uint32_t b, uint32_t m, uint32_t n_esc,
                           uint32_t rec_bytes, uint4 (&v)[kPer]) {
  const int t = ctid();
  const uint8_t* st = stage8(s);
  if (mode == 0) {
    const uint32_t n16 = (rec_bytes - 16u) / 16u;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const uint32_t c = t + kCT * k;
      v[k] = c < n16 ? s.stage[1 + c] : make_uint4(0, 0, 0, 0);
    }
    // padding after the m words must be zero
    bool bad = false;
    for (uint32_t i = 16u + 2u * m + t; i < rec_bytes; i += kCT) bad |= st[i] != 0;
    const bool any_bad = __syncthreads_or(bad);
    if (!any_bad && m != kB) {  // clear lanes past m so callers see zeros there
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const uint32_t e0 = 8u * (t + kCT * k);
        uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
    #pragma unroll
        for (uint32_t i = 0; i < 8; ++i)
          if (e0 + i >= m) w4[i >> 1] &= (i & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        v[k] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
    return !any_bad;
  }
  switch (b) {
    case 1: return read_coded<1>(s, n_esc, v);
    case 2: return read_coded<2>(s, n_esc, v);
    case 3: return read_coded<3>(s, n_esc, v);
    case 4: return read_coded<4>(s, n_esc, v);
    case 5: return read_coded<5>(s, n_esc, v);
    case 6: return read_coded<6>(s, n_esc, v);
    default: return read_coded<7>(s, n_esc, v);
  }
}

}  // inline namespace HC_CODEC_TID_NS
}  // namespace codec
}  // namespace hc
