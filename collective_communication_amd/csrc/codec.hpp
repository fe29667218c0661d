// codec.hpp -- one HCZ1 block (16384 bf16 = 32 KB) per 256-thread workgroup.
//
// The method is the exponent coder of "CCCL: In-GPU Compression-Coupled
// Collective Communication": section 4.1 (a bf16 word splits into sign,
// exponent and fraction; sign and fraction are sent as they are, the skewed
// 8-bit exponent is coded from a frequency table), section 4.3 (each block
// builds its own table; every symbol gets a fixed-length code) and section
// 4.4 (the block writes its output in one pass, no temporary buffers).  Byte
// format: see include/hc.h.
//
// gfx950 mapping.  Thread t of the workgroup owns the eight 16-byte chunks
// c = t + 256k (k = 0..7) of the block, eight consecutive elements each, so
// every global load and store of a wave is a contiguous 1 KB.  A chunk is
// exactly one byte of each code plane, which makes plane packing a bit-matrix
// transpose inside one register pair.  The record is assembled in LDS
// (<= 32784 bytes) and leaves with 16-byte stores.
//   histogram : LDS atomics into 32 replicated, bank-skewed sub-histograms
//               (two 16-bit bins per word) held in the staging buffer, then
//               one thread per exponent sums its 32 copies
//   ranking   : occurring exponents are compacted (ballot + popcount) and
//               each ranks itself against that short list of keys (count
//               desc, exponent asc); absent exponents rank after them in order
//   b choice  : wave 0 prefix-sums the ranked counts and takes the min of
//               the seven candidate sizes (ties to the smaller b)
//   escapes   : per-chunk counts, workgroup exclusive scan (wave shuffles +
//               one LDS exchange), escaped exponent bytes written in order
#pragma once

#include "common.hpp"

namespace hc {
namespace codec {

constexpr uint32_t kB = 16384;                  // elements per block
constexpr uint32_t kChunks = kB / 8;            // 16-byte chunks per block
constexpr int kPer = kChunks / kThreads;        // chunks per thread (8)
constexpr uint32_t kPlaneBytes = kB / 8;        // one code plane
constexpr uint32_t kRawFull = 16 + 2 * kB;      // raw record of a full block
constexpr uint32_t kStage16 = kRawFull / 16;    // 2049 uint4 of LDS staging
constexpr uint32_t kMagic = 0x315A4348u;

struct Plan {
  uint32_t mode;       // 0 raw, 1 coded
  uint32_t b;          // code bits (coded)
  uint32_t K;          // dictionary entries = escape code
  uint32_t n_esc;
  uint32_t rec_bytes;
  uint32_t m;          // elements in the block
};

struct Smem {
  uint4 stage[kStage16];         // the record being built or read
  uint32_t key[256];             // (count << 8) | (255 - exponent) of occurring exponents
  uint32_t cbr[256];             // count by rank
  uint8_t code_of[256];          // exponent -> code
  uint32_t wsum[kWaves][4];      // per-wave escape-count totals (scan)
  uint32_t plan[8];
  uint64_t misc[2];
};

__device__ __forceinline__ uint8_t* stage8(Smem& s) { return reinterpret_cast<uint8_t*>(s.stage); }

__device__ __forceinline__ uint32_t dict_bytes(uint32_t b) { return (1u << b) < 16u ? 16u : (1u << b); }
__device__ __forceinline__ uint32_t coded_bytes(uint32_t b, uint32_t n_esc) {
  return 16u + dict_bytes(b) + kPlaneBytes * b + kB + ((n_esc + 15u) & ~15u);
}
__device__ __forceinline__ uint32_t raw_bytes(uint32_t m) { return 16u + ((2u * m + 15u) & ~15u); }
__device__ __forceinline__ uint32_t planes_off(uint32_t b) { return 16u + dict_bytes(b); }
__device__ __forceinline__ uint32_t sm_off(uint32_t b) { return planes_off(b) + kPlaneBytes * b; }
__device__ __forceinline__ uint32_t esc_off(uint32_t b) { return sm_off(b) + kB; }

// 8x8 bit-matrix transpose of a 64-bit word (byte r, bit c) -> (byte c, bit
// r), by three rounds of delta swaps over 1x1, 2x2 and 4x4 sub-blocks (the
// recursive block transpose described in Hacker's Delight, section 7-3).
// The transpose is its own inverse.
__device__ __forceinline__ uint64_t transpose8(uint64_t x) {
  uint64_t t;
  t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
  x = x ^ t ^ (t << 7);
  t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
  x = x ^ t ^ (t << 14);
  t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
  x = x ^ t ^ (t << 28);
  return x;
}

// Sign and fraction of the two bf16 halves of w as two bytes:
// byte = sign << 7 | fraction.
__device__ __forceinline__ uint32_t sm_pair(uint32_t w) {
  const uint32_t t = w & 0x807F807Fu;
  return (t & 0x7Fu) | ((t >> 8) & 0x7F80u) | ((t >> 16) & 0x8000u);
}

__device__ __forceinline__ uint32_t exp_lo(uint32_t w) { return (w >> 7) & 0xFFu; }
__device__ __forceinline__ uint32_t exp_hi(uint32_t w) { return (w >> 23) & 0xFFu; }

__device__ __forceinline__ uint32_t chunk_elem_word(const uint4& v, int i) {
  const uint32_t w = (i < 2) ? v.x : (i < 4) ? v.y : (i < 6) ? v.z : v.w;
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Exponent histogram layout during planning: kHistCopies sub-histograms in
// the (not yet used) staging buffer, lane l of every wave adding into copy
// l % 32, two 16-bit bins per 32-bit word.  The odd word stride puts the
// copies of one bin in different LDS banks, so the lanes of a wave that hold
// the same exponent (most of them, for trained-model data) do not collide.
constexpr uint32_t kHistCopies = 32;
constexpr uint32_t kHistStride = 129;   // words per copy (128 + 1)

// Inclusive wave64 prefix sum of four packed counters.
__device__ __forceinline__ uint4 wave_incl_scan4(uint4 v) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t x = __shfl_up(v.x, d, 64), y = __shfl_up(v.y, d, 64);
    const uint32_t z = __shfl_up(v.z, d, 64), w = __shfl_up(v.w, d, 64);
    if (lane >= d) { v.x += x; v.y += y; v.z += z; v.w += w; }
  }
  return v;
}

__device__ __forceinline__ uint32_t field16(const uint4& v, int k) {
  const uint32_t w = (k < 2) ? v.x : (k < 4) ? v.y : (k < 6) ? v.z : v.w;
  return (k & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Workgroup exclusive scan of per-(thread, k) counts cnt[k] (each <= 8) in
// element index order (chunk c = t + 256k, so k-major, then thread).  Returns
// for each k the number of counted elements before this thread's chunk k.
// Counters travel as 16-bit fields, two per 32-bit lane of a uint4.
__device__ __forceinline__ void block_excl_scan8(const uint32_t (&cnt)[kPer], uint32_t (&excl)[kPer],
                                                 Smem& s) {
  const uint4 mine = make_uint4(cnt[0] | (cnt[1] << 16), cnt[2] | (cnt[3] << 16),
                                cnt[4] | (cnt[5] << 16), cnt[6] | (cnt[7] << 16));
  const uint4 incl = wave_incl_scan4(mine);
  const int wave = threadIdx.x >> 6;
  if (__lane_id() == 63) {
    s.wsum[wave][0] = incl.x; s.wsum[wave][1] = incl.y;
    s.wsum[wave][2] = incl.z; s.wsum[wave][3] = incl.w;
  }
  __syncthreads();
  uint4 before = make_uint4(0, 0, 0, 0), total = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint4 t = make_uint4(s.wsum[w][0], s.wsum[w][1], s.wsum[w][2], s.wsum[w][3]);
    if (w < wave) { before.x += t.x; before.y += t.y; before.z += t.z; before.w += t.w; }
    total.x += t.x; total.y += t.y; total.z += t.z; total.w += t.w;
  }
  uint32_t base = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t in_wave = field16(incl, k) - field16(mine, k);
    excl[k] = base + field16(before, k) + in_wave;
    base += field16(total, k);
  }
}

// Loads a block's elements: thread t gets chunks t + 256k.  Elements at or
// past m read as zero.
__device__ __forceinline__ void load_block(const uint16_t* src, uint32_t m, uint4 (&v)[kPer]) {
  const int t = threadIdx.x;
  if (m == kB) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = ld16(src + 8 * (t + kThreads * k));
    return;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t e0 = 8u * (t + kThreads * k);
    uint32_t w[4] = {0, 0, 0, 0};
    for (uint32_t i = 0; i < 8; ++i)
      if (e0 + i < m) w[i >> 1] |= (uint32_t)src[e0 + i] << (16 * (i & 1));
    v[k] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Stores a block's elements (first m only).
__device__ __forceinline__ void store_block(uint16_t* dst, uint32_t m, const uint4 (&v)[kPer]) {
  const int t = threadIdx.x;
  if (m == kB) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) st16(dst + 8 * (t + kThreads * k), v[k]);
    return;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t e0 = 8u * (t + kThreads * k);
    for (uint32_t i = 0; i < 8; ++i)
      if (e0 + i < m) dst[e0 + i] = (uint16_t)chunk_elem_word(v[k], (int)i);
  }
}

// Phase 1 of encoding: histogram, ranking, the choice of b and the record
// size.  Leaves code_of[] and the plan in LDS; returns the plan (uniform).
__device__ Plan plan_block(const uint4 (&v)[kPer], uint32_t m, Smem& s) {
  const int t = threadIdx.x;
  Plan p;
  p.m = m;
  if (m != kB) {  // partial blocks travel raw
    p.mode = 0; p.b = 0; p.K = 0; p.n_esc = 0; p.rec_bytes = raw_bytes(m);
    return p;
  }
  uint32_t* sub = reinterpret_cast<uint32_t*>(s.stage);
  for (uint32_t i = t; i < kHistCopies * kHistStride; i += kThreads) sub[i] = 0;
  __syncthreads();
  {
    uint32_t* mine = sub + (__lane_id() & (kHistCopies - 1)) * kHistStride;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t e0 = exp_lo(w4[q]), e1 = exp_hi(w4[q]);
        atomicAdd(&mine[e0 >> 1], 1u << ((e0 & 1u) << 4));
        atomicAdd(&mine[e1 >> 1], 1u << ((e1 & 1u) << 4));
      }
    }
  }
  __syncthreads();
  uint32_t cnt = 0;
#pragma unroll 8
  for (uint32_t c = 0; c < kHistCopies; ++c) cnt += (sub[c * kHistStride + (t >> 1)] >> ((t & 1) << 4)) & 0xFFFFu;
  // Rank = position in (count desc, exponent asc).  Only exponents that occur
  // need comparisons: they are compacted into a short list of keys; an
  // exponent that never occurs ranks after all that do, in exponent order.
  const uint32_t key = (cnt << 8) | (255u - (uint32_t)t);
  const uint64_t nzmask = __ballot(cnt > 0);
  const uint32_t wave = (uint32_t)t >> 6;
  const uint32_t below = (uint32_t)__popcll(nzmask & ((1ull << __lane_id()) - 1ull));
  if (__lane_id() == 0) s.wsum[wave][0] = (uint32_t)__popcll(nzmask);
  __syncthreads();
  uint32_t before = 0, nz_total = 0;
#pragma unroll
  for (uint32_t w = 0; w < (uint32_t)kWaves; ++w) {
    const uint32_t c = s.wsum[w][0];
    before += w < wave ? c : 0;
    nz_total += c;
  }
  const uint32_t nz_below = before + below;
  if (cnt > 0) s.key[nz_below] = key;
  __syncthreads();
  uint32_t rank;
  if (cnt > 0) {
    rank = 0;
    for (uint32_t i = 0; i < nz_total; ++i) rank += s.key[i] > key;
  } else {
    rank = nz_total + ((uint32_t)t - nz_below);
  }
  s.cbr[rank] = cnt;
  __syncthreads();
  if (t < 64) {
    // cover(K) = sum of the K largest counts, K = 2^b - 1.  Lane l holds
    // ranks 2l and 2l+1; after the inclusive scan S_l covers ranks <= 2l+1,
    // and cover(2^b - 1) = S_l - cbr[2l+1] at lane l = 2^(b-1) - 1.
    const uint32_t a = s.cbr[2 * t], bb = s.cbr[2 * t + 1];
    uint32_t S = a + bb;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t x = __shfl_up(S, d, 64);
      if (t >= d) S += x;
    }
    const uint32_t cover = S - bb;
    // candidate key: size, then b (so the smaller b wins a tie), then n_esc
    uint64_t cand = ~0ull;
    const uint32_t l1 = (uint32_t)t + 1;
    if ((l1 & (l1 - 1)) == 0) {  // t = 2^(b-1) - 1 for b = 1..7
      const uint32_t b = 32 - __clz(l1);
      const uint32_t n_esc = kB - cover;
      cand = ((uint64_t)coded_bytes(b, n_esc) << 32) | ((uint64_t)b << 24) | n_esc;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const uint64_t o = __shfl_xor(cand, d, 64);
      cand = o < cand ? o : cand;
    }
    if (t == 0) {
      const uint32_t size = (uint32_t)(cand >> 32);
      const uint32_t b = (uint32_t)(cand >> 24) & 0xFFu;
      const uint32_t n_esc = (uint32_t)cand & 0xFFFFFFu;
      if (size < kRawFull) {
        s.plan[0] = 1; s.plan[1] = b; s.plan[2] = (1u << b) - 1; s.plan[3] = n_esc; s.plan[4] = size;
      } else {
        s.plan[0] = 0; s.plan[1] = 0; s.plan[2] = 0; s.plan[3] = 0; s.plan[4] = kRawFull;
      }
    }
  }
  __syncthreads();
  p.mode = s.plan[0]; p.b = s.plan[1]; p.K = s.plan[2]; p.n_esc = s.plan[3]; p.rec_bytes = s.plan[4];
  if (p.mode == 1) {
    s.code_of[t] = (uint8_t)(rank < p.K ? rank : p.K);
    if (rank < p.K) stage8(s)[16 + rank] = (uint8_t)t;        // dictionary entry
    else if (rank < dict_bytes(p.b)) stage8(s)[16 + rank] = 0;  // dictionary padding
  }
  __syncthreads();
  return p;
}

// Phase 2 of encoding: writes the record for plan p into the LDS staging
// buffer.  Ends with a barrier.
__device__ void write_block(const uint4 (&v)[kPer], const Plan& p, Smem& s) {
  const int t = threadIdx.x;
  uint8_t* st = stage8(s);
  if (t == 0) {
    uint32_t* h = reinterpret_cast<uint32_t*>(st);
    h[0] = p.mode | (p.b << 8);
    h[1] = p.m;
    h[2] = p.n_esc;
    h[3] = p.rec_bytes;
  }
  if (p.mode == 0) {
    const uint32_t n16 = (p.rec_bytes - 16u) / 16u;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const uint32_t c = t + kThreads * k;
      if (c < n16) s.stage[1 + c] = v[k];
    }
    __syncthreads();
    return;
  }
  const uint32_t b = p.b, K = p.K;
  const uint32_t poff = planes_off(b), soff = sm_off(b), eoff = esc_off(b);
  uint32_t escmask[kPer], cnt[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t c = t + kThreads * k;
    const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
    uint32_t lo = 0, hi = 0, em = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t c0 = s.code_of[exp_lo(w4[q])];
      const uint32_t c1 = s.code_of[exp_hi(w4[q])];
      em |= (uint32_t)(c0 == K) << (2 * q);
      em |= (uint32_t)(c1 == K) << (2 * q + 1);
      const uint32_t pair = c0 | (c1 << 8);
      if (q < 2) lo |= pair << (16 * q);
      else hi |= pair << (16 * (q - 2));
    }
    const uint64_t planes = transpose8(((uint64_t)hi << 32) | lo);
    for (uint32_t j = 0; j < b; ++j) st[poff + j * kPlaneBytes + c] = (uint8_t)(planes >> (8 * j));
    const uint32_t sm01 = sm_pair(w4[0]) | (sm_pair(w4[1]) << 16);
    const uint32_t sm23 = sm_pair(w4[2]) | (sm_pair(w4[3]) << 16);
    *reinterpret_cast<uint2*>(st + soff + 8 * c) = make_uint2(sm01, sm23);
    escmask[k] = em;
    cnt[k] = __popc(em);
  }
  if (p.n_esc) {
    uint32_t excl[kPer];
    block_excl_scan8(cnt, excl, s);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      uint32_t em = escmask[k], pos = excl[k];
      const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
      while (em) {
        const int i = __ffs(em) - 1;
        em &= em - 1;
        const uint32_t w = w4[i >> 1];
        st[eoff + pos++] = (uint8_t)((i & 1) ? exp_hi(w) : exp_lo(w));
      }
    }
    const uint32_t pad_end = (p.n_esc + 15u) & ~15u;
    if ((uint32_t)t < pad_end - p.n_esc) st[eoff + p.n_esc + t] = 0;
  }
  __syncthreads();
}

// Copies a staged record (rec_bytes, a multiple of 16) to global memory.
__device__ __forceinline__ void copy_out(const Smem& s, uint8_t* dst, uint32_t rec_bytes) {
  const uint32_t n16 = rec_bytes / 16u;
  for (uint32_t i = threadIdx.x; i < n16; i += kThreads) st16(dst + 16 * i, s.stage[i]);
}

// Copies a record from global memory into the staging buffer.
__device__ __forceinline__ void copy_in(Smem& s, const uint8_t* src, uint32_t rec_bytes) {
  const uint32_t n16 = rec_bytes / 16u;
  for (uint32_t i = threadIdx.x; i < n16; i += kThreads) s.stage[i] = ld16(src + 16 * i);
}

// Decodes the staged record (header already validated for mode, b, m,
// rec_bytes) into v.  Returns false (uniform) when the escape count or a
// padding byte disagrees with the format.  Ends with a barrier.
__device__ bool read_block(Smem& s, uint32_t mode, uint32_t b, uint32_t m, uint32_t n_esc,
                           uint32_t rec_bytes, uint4 (&v)[kPer]) {
  const int t = threadIdx.x;
  const uint8_t* st = stage8(s);
  if (mode == 0) {
    const uint32_t n16 = (rec_bytes - 16u) / 16u;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const uint32_t c = t + kThreads * k;
      v[k] = c < n16 ? s.stage[1 + c] : make_uint4(0, 0, 0, 0);
    }
    // padding after the m words must be zero
    bool bad = false;
    for (uint32_t i = 16u + 2u * m + t; i < rec_bytes; i += kThreads) bad |= st[i] != 0;
    const bool any_bad = __syncthreads_or(bad);
    if (!any_bad && m != kB) {  // clear lanes past m so callers see zeros there
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const uint32_t e0 = 8u * (t + kThreads * k);
        uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        for (uint32_t i = 0; i < 8; ++i)
          if (e0 + i >= m) w4[i >> 1] &= (i & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        v[k] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
    return !any_bad;
  }
  const uint32_t K = (1u << b) - 1u;
  const uint32_t poff = planes_off(b), soff = sm_off(b), eoff = esc_off(b);
  bool bad = false;
  // dictionary padding must be zero
  if ((uint32_t)t >= K && (uint32_t)t < dict_bytes(b)) bad |= st[16 + t] != 0;
  uint32_t codes_lo[kPer], codes_hi[kPer], cnt[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t c = t + kThreads * k;
    uint64_t x = 0;
    for (uint32_t j = 0; j < b; ++j) x |= (uint64_t)st[poff + j * kPlaneBytes + c] << (8 * j);
    const uint64_t codes = transpose8(x);
    codes_lo[k] = (uint32_t)codes;
    codes_hi[k] = (uint32_t)(codes >> 32);
    uint32_t n = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      n += ((codes_lo[k] >> (8 * i)) & 0xFFu) == K;
      n += ((codes_hi[k] >> (8 * i)) & 0xFFu) == K;
    }
    cnt[k] = n;
  }
  uint32_t excl[kPer];
  block_excl_scan8(cnt, excl, s);
  // total escapes = excl of the last chunk of the last thread + its count
  uint32_t total = 0;
  if (t == kThreads - 1) total = excl[kPer - 1] + cnt[kPer - 1];
  if (t == kThreads - 1) s.plan[7] = total;
  // escape padding must be zero
  const uint32_t pad_end = (n_esc + 15u) & ~15u;
  if ((uint32_t)t < pad_end - n_esc) bad |= st[eoff + n_esc + t] != 0;
  __syncthreads();
  const bool count_ok = s.plan[7] == n_esc;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t c = t + kThreads * k;
    const uint2 smv = *reinterpret_cast<const uint2*>(st + soff + 8 * c);
    uint32_t pos = excl[k];
    uint32_t w4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t cw = q < 2 ? codes_lo[k] : codes_hi[k];
      const uint32_t code0 = (cw >> (16 * (q & 1))) & 0xFFu;
      const uint32_t code1 = (cw >> (16 * (q & 1) + 8)) & 0xFFu;
      uint32_t e0, e1;
      if (code0 == K) { e0 = (count_ok && pos < n_esc) ? st[eoff + pos] : 0; ++pos; }
      else e0 = st[16 + code0];
      if (code1 == K) { e1 = (count_ok && pos < n_esc) ? st[eoff + pos] : 0; ++pos; }
      else e1 = st[16 + code1];
      const uint32_t smw = (q < 2 ? smv.x : smv.y) >> (16 * (q & 1));
      const uint32_t s0 = smw & 0xFFu, s1 = (smw >> 8) & 0xFFu;
      const uint32_t lo = ((s0 & 0x80u) << 8) | (e0 << 7) | (s0 & 0x7Fu);
      const uint32_t hi = ((s1 & 0x80u) << 8) | (e1 << 7) | (s1 & 0x7Fu);
      w4[q] = lo | (hi << 16);
    }
    v[k] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
  const bool any_bad = __syncthreads_or(bad || !count_ok);
  return !any_bad;
}

}  // namespace codec
}  // namespace hc
