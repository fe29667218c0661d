// entropy_kernels.hip -- HCE1, the bf16 codec with an entropy-coded exponent,
// for gfx950.
//
// "CCCL: In-GPU Compression-Coupled Collective Communication", section 4.1
// codes the bf16 exponent from a frequency table and keeps sign and fraction
// raw; the CCCL core uses fixed-length codes, and section 6.5 compares it with
// an entropy coder whose output is smaller by under 7%.  HCE1 is that
// comparison built in the same container: each full block of 16,384 elements
// codes its exponents with its own canonical Huffman code, lengths at most 12
// bits, and keeps the sign/fraction byte plane raw.  The full format is
// stated in include/hc.h (hc_compress_bf16_entropy).
//
// Parallel layout.  A block is read by 64 lanes of 256 elements (lane j:
// elements 64 i + j, step i).  Each lane's codes form one bit stream cut into
// 32-bit words, and the words of all lanes are stored in the order in which a
// decoder running the 64 lanes in lockstep takes them: a lane takes its next
// word when the bits it holds do not contain its next code, lanes in order
// within a step.  So no per-lane offsets are stored, and each lane pads only
// its last word.
//
// compress: one workgroup of 512 threads per block, block = workgroup index,
// the record published and placed by the decoupled look-back of the
// fixed-length encoder (one read of the input, one write of the output).
// After the histogram, one thread builds the Huffman lengths (two queues over
// the exponents sorted by count); the canonical codes come out in parallel.
// The eight waves then each code 32 steps of all 64 lanes: a first pass adds
// up the bits of every (step segment, lane), which fixes each segment's start
// bit in every lane and the number of words taken before it, so the record
// size is known and published before any word is written; the second pass
// writes the words at their final positions, and the one word that two
// segments of a lane share is merged afterwards.
//
// decompress: one wave per block (the 64 lanes are the 64 streams).  The
// code lengths give a two-level table (12-bit window -> symbol, length) in
// LDS; the next 128 words of the record sit in two registers across the
// wave and a lane takes its word by a lane shuffle, so the only memory on
// the per-step chain is the table read.
#include "codec.hpp"
#include "launch.hpp"
#include "lookback.hpp"
#include "schedule.hpp"

namespace hc {

using namespace codec;

namespace {

constexpr uint32_t kHceMagic = 0x31454348u;   // "HCE1"
constexpr uint32_t kLmax = 12;                  // longest code
constexpr uint32_t kLanes = 64;                 // bit streams per block
constexpr uint32_t kSteps = kB / kLanes;        // codes per stream (256)
constexpr uint32_t kSegs = kCW;                 // encoder: one wave per segment of steps
constexpr uint32_t kSegSteps = kSteps / kSegs;  // 32
constexpr uint32_t kSmOff = 144;                // sign/fraction plane
constexpr uint32_t kWordsOff = kSmOff + kB;     // 16,528: the interleaved words
constexpr uint32_t kMaxWords = 4060;            // most words of a record smaller than the raw one

__host__ __device__ constexpr uint32_t hce_coded_bytes(uint32_t n_words) {
  return kWordsOff + ((4u * n_words + 15u) & ~15u);
}
static_assert(hce_coded_bytes(kMaxWords) < kRawFull && hce_coded_bytes(kMaxWords + 1) >= kRawFull,
              "kMaxWords is the largest coded record below the raw size");
static_assert(kSegSteps == 32, "one bit per step of a segment in a 32-bit mask");

// Huffman scratch inside the record's words region (free until the words are
// written): weights of leaves and merged nodes, parents, leaves in increasing
// (count, decreasing exponent) order, sort keys, leaf lengths.
constexpr uint32_t kHwOff = kWordsOff;              // u32 [511]
constexpr uint32_t kHparOff = kWordsOff + 2048;     // u16 [511]
constexpr uint32_t kSymOff = kWordsOff + 3072;      // u8 [256]
constexpr uint32_t kKeyOff = kWordsOff + 3328;      // u32 [256]
constexpr uint32_t kLeafLenOff = kWordsOff + 4352;  // u8 [256]
static_assert(kLeafLenOff + 256 <= kRawFull, "scratch fits the staging buffer");

struct HceEncSmem {
  uint4 stage[kStage16 + 1];        // sub-histograms, then the record
  uint32_t enc[256];                // exponent -> code bits in stream order | length << 16
  uint32_t seg[kSegs][kLanes];      // bits of each (segment, lane); then carried words
  uint16_t lastpos[kSegs][kLanes];  // position of each (segment, lane)'s unfinished last word
  uint8_t len[256];                 // exponent -> code length (0: absent)
  uint32_t cbl[4][kLmax + 1];       // per owner wave: codes of each length
  uint32_t wcount[4];
  uint32_t plan[8];
  uint64_t misc[2];
};

__device__ __forceinline__ uint32_t lanemask_lt_count(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Word k (0..15) of the packed elements.
__device__ __forceinline__ uint32_t word_of(const uint4 (&v)[kPer], int k) {
  const uint4& q = v[k >> 2];
  switch (k & 3) {
    case 0: return q.x;
    case 1: return q.y;
    case 2: return q.z;
    default: return q.w;
  }
}

// The thread's 32 elements: 2048 seg + 64 i + lane, i = 0..31 (its lane's
// steps 32 seg + i), two per word, element i in half i & 1 of word i / 2.
// Elements at or past m read as 0.
__device__ __forceinline__ void load_lane_steps(const uint16_t* src, uint32_t m, uint32_t seg, uint32_t lane,
                                                uint4 (&v)[kPer]) {
  uint32_t w[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t i0 = 2048u * seg + 64u * (2u * k) + lane, i1 = i0 + 64u;
    const uint32_t lo = i0 < m ? src[i0] : 0u, hi = i1 < m ? src[i1] : 0u;
    w[k] = lo | (hi << 16);
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) v[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
}

// The same elements of a full block, through LDS: each lane moves 16-byte
// pieces of the block straight into the staging buffer (four per thread, no
// registers held), then reads its 32 elements there.  Measured on MI355X for
// 2^28 elements: 0.41 ms per call against 0.52 ms with the 32 two-byte global
// loads per lane of load_lane_steps.  Ends with a barrier: the staging buffer
// is free again.
__device__ __forceinline__ void load_block_lanes(const uint16_t* src, uint32_t seg, uint32_t lane, HceEncSmem& s,
                                                 uint4 (&v)[kPer]) {
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t c0 = kCT * k + 64u * seg;   // first 16-byte chunk of this wave's 1 KB
    __builtin_amdgcn_global_load_lds(src + 8 * (c0 + lane),
                                     (__attribute__((address_space(3))) void*)&s.stage[c0], 16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);   // LDS DMA completes on the vector memory counter
  __syncthreads();
  const uint16_t* e16 = reinterpret_cast<const uint16_t*>(s.stage);
  uint32_t w[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t i0 = 2048u * seg + 64u * (2u * k) + lane;
    w[k] = (uint32_t)e16[i0] | ((uint32_t)e16[i0 + 64u] << 16);
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) v[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
  __syncthreads();
}

__device__ __forceinline__ uint32_t elem_of(const uint4 (&v)[kPer], int i) {
  const uint32_t w = word_of(v, i >> 1);
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Huffman depths of up to 64 leaves (weights lw: leaf `lane`, increasing)
// in the registers of one wave: the same two-queue construction as the LDS
// loop below, with the fronts read by readlane and the merged nodes' weights
// and parents written by writelane.  Returns leaf `lane`'s depth.
// v with lane `at` (uniform) replaced by x.
__device__ __forceinline__ uint32_t set_lane(uint32_t v, uint32_t at, uint32_t x) {
  return __lane_id() == at ? x : v;
}

__device__ __forceinline__ uint32_t huffman_depths_wave(uint32_t lw, uint32_t n) {
  // Queue fronts as scalars: wl the next leaf's weight, wn the next merged
  // node's, kInf for an empty queue (at least two items remain at every
  // pick, so a pick never meets two empty queues).  Every branch below is
  // on wave-uniform values.
  constexpr uint32_t kInf = 0xFFFFFFFFu;
  uint32_t nw = 0, lpar = 0, npar = 0;   // merged node k's weight; parents (merged-node numbers)
  uint32_t leaf = 0, node = 0, made = 0;
  uint32_t wl = lane_read(lw, 0), wn = kInf;
  for (uint32_t k = 0; k + 1 < n; ++k) {
    uint32_t sum = 0;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      leaf = first_lane_read(leaf);   // keeps the counter scalar
      if (wl <= wn) {                 // a leaf; a leaf on a tie
        sum += wl;
        lpar = set_lane(lpar, leaf, made);
        ++leaf;
        wl = leaf < n ? lane_read(lw, leaf) : kInf;
      } else {
        sum += wn;
        npar = set_lane(npar, node, made);
        ++node;
        wn = node < made ? lane_read(nw, node) : kInf;
      }
    }
    nw = set_lane(nw, made, sum);
    if (node == made) wn = sum;   // the new node is the front of its queue
    ++made;
  }
  // depths of the merged nodes, root (made - 1) first: a parent is made after its children
  uint32_t nd = 0;
  for (int32_t j = (int32_t)made - 2; j >= 0; --j) {
    const uint32_t pd = lane_read(nd, lane_read(npar, j));
    nd = set_lane(nd, (uint32_t)j, pd + 1u);
  }
  return __shfl(nd, (int)lpar, 64) + 1u;
}

// The whole code of a block with 2..64 exponents present, built by one wave
// with no workgroup barrier: the same lengths and codes as the workgroup
// path of build_code below, which serves every other count.  s.enc holds
// the counts by exponent on entry; leaves s.enc, s.len and the length table.
//   1. Present exponents as keys (count << 8 | 255 - exponent), one per lane
//      in exponent order; a key's rank among them (greater keys) makes it
//      leaf n - 1 - rank, leaves in increasing (count, decreasing exponent).
//   2. The two-queue Huffman depths (huffman_depths_wave), cut to kLmax.
//   3. While the Kraft sum exceeds 1, the longest code shorter than kLmax
//      grows by a bit (ties: the lowest leaf, i.e. the lightest).
//   4. Canonical codes: a code's place in (length, exponent) order is the
//      number of (length << 8 | exponent) keys below its own; the first code
//      of length L is (first of L - 1 + codes of L - 1) << 1.
__device__ void build_code_wave(uint32_t n, HceEncSmem& s) {
  const uint32_t lane = __lane_id();
  uint32_t* keys = reinterpret_cast<uint32_t*>(stage8(s) + kKeyOff);
  uint32_t c[4];
  uint64_t pm[4];
  uint32_t before = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    c[k] = s.enc[lane + 64u * k];
    pm[k] = __ballot(c[k] > 0);
    if (c[k] > 0) keys[before + lanemask_lt_count(pm[k])] = (c[k] << 8) | (255u - (lane + 64u * k));
    before += (uint32_t)__popcll(pm[k]);
  }
  __builtin_amdgcn_wave_barrier();   // one wave: LDS accesses stay in program order
  const bool live = lane < n;
  const uint32_t key = live ? keys[lane] : 0u;
  uint32_t above = 0;
  for (uint32_t j = 0; j < n; ++j) above += lane_read(key, j) > key ? 1u : 0u;
  const uint32_t a = n - 1u - above;              // this key's leaf
  // leaf order: weights and exponents through LDS (the same wave writes and reads)
  uint32_t* hw = reinterpret_cast<uint32_t*>(stage8(s) + kHwOff);
  uint8_t* sym_asc = stage8(s) + kSymOff;
  if (live) {
    hw[a] = key >> 8;
    sym_asc[a] = (uint8_t)(255u - (key & 0xFFu));
  }
  __builtin_amdgcn_wave_barrier();
  const uint32_t lw = live ? hw[lane] : 0u;
  const uint32_t sym = live ? sym_asc[lane] : 0u;
  const uint32_t depth = huffman_depths_wave(lw, n);
  uint32_t len = live ? (depth > kLmax ? kLmax : depth) : 0u;
  if (__ballot(live && depth > kLmax)) {
    uint32_t kraft = wave_sum(live ? 1u << (kLmax - len) : 0u);
    while (kraft > (1u << kLmax)) {
      uint32_t at = 64u, bl = 0;
      for (uint32_t L = kLmax - 1u; L >= 1u && at == 64u; --L) {
        const uint64_t m = __ballot(live && len == L);
        if (m) { at = (uint32_t)__builtin_ctzll(m); bl = L; }
      }
      if (at == 64u) break;                       // every code is kLmax long: cannot happen with <= 64 leaves
      if (lane == at) ++len;
      kraft -= 1u << (kLmax - bl - 1u);
    }
  }
  // canonical codes
  const uint32_t key2 = live ? (len << 8) | sym : 0xFFFFFFFFu;
  uint32_t place = 0;
  for (uint32_t j = 0; j < n; ++j) place += lane_read(key2, j) < key2 ? 1u : 0u;
  uint32_t base = 0;          // first code of this length minus the codes before it in canonical order
  {
    uint32_t code = 0, prev = 0, idx = 0;
#pragma unroll
    for (uint32_t L = 1; L <= kLmax; ++L) {
      code = (code + prev) << 1;
      const uint32_t cntL = (uint32_t)__popcll(__ballot(live && len == L));
      if (len == L) base = code - idx;
      prev = cntL;
      idx += cntL;
    }
  }
  const uint32_t code = base + place;
  // tables by exponent: clear, then the present ones (one wave: in order)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s.enc[lane + 64u * k] = 0;
    s.len[lane + 64u * k] = 0;
  }
  if (live) {
    s.enc[sym] = (__builtin_bitreverse32(code) >> (32u - len)) | (len << 16);
    s.len[sym] = (uint8_t)len;
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t b = lane + 64u * k;
    stage8(s)[16 + b] = (uint8_t)(s.len[2 * b] | (s.len[2 * b + 1] << 4));
  }
}

// Code lengths (Huffman, limited to kLmax) and canonical codes for the
// exponent counts (thread t < 256 holds the count of exponent t).  Leaves
// s.enc, s.len and the record's length table (bytes 16..143); returns the
// number of exponents present.  Starts and ends with a barrier.  `others`
// runs on the waves that do not build the code while one wave does (with 2
// to 64 exponents present), else after the code is built.
template <class Others>
__device__ uint32_t build_code(uint32_t cnt, HceEncSmem& s, Others others) {
  const uint32_t t = threadIdx.x, lane = t & 63u, wave = t >> 6;
  uint32_t* hw = reinterpret_cast<uint32_t*>(stage8(s) + kHwOff);
  uint16_t* hpar = reinterpret_cast<uint16_t*>(stage8(s) + kHparOff);
  uint8_t* sym_asc = stage8(s) + kSymOff;
  uint32_t* keys = reinterpret_cast<uint32_t*>(stage8(s) + kKeyOff);
  uint8_t* leaf_len = stage8(s) + kLeafLenOff;
  const bool owner = t < 256u;
  const bool present = owner && cnt > 0;
  const uint64_t pm = __ballot(present);
  if (owner && lane == 0) s.wcount[wave] = (uint32_t)__popcll(pm);
  if (owner) s.enc[t] = cnt;
  if (t == 0) s.plan[5] = 0;
  __syncthreads();
  uint32_t before = 0, n = 0;
#pragma unroll
  for (uint32_t w = 0; w < 4; ++w) {
    const uint32_t c = s.wcount[w];
    before += w < wave ? c : 0u;
    n += c;
  }
  if (n >= 2 && n <= 64) {
    if (first_lane_read(t) < 64u) {   // wave 0, as a uniform branch
      build_code_wave(n, s);
    } else {
      others();
    }
    __syncthreads();
    if (first_lane_read(t) < 64u) others();
    return n;
  }
  // Occurring exponents, ranked by (count, then exponent descending):
  // leaf a of the Huffman construction is the a-th lightest.
  const uint32_t key = (cnt << 8) | (255u - t);
  if (present) keys[before + lanemask_lt_count(pm)] = key;
  if (owner) s.len[t] = 0;
  __syncthreads();
  if (present) {
    uint32_t above = 0;
    for (uint32_t j = 0; j < n; ++j) above += keys[j] > key;
    const uint32_t a = n - 1u - above;
    sym_asc[a] = (uint8_t)t;
    hw[a] = cnt;
  }
  __syncthreads();
  // Two queues: the next leaf and the next merged node; the lighter goes
  // first, a leaf on a tie.  Merged nodes are made in increasing weight.
  if (t == 0 && n >= 2) {
    uint32_t leaf = 0, node = n, made = n;
    for (uint32_t k = 0; k + 1 < n; ++k) {
      uint32_t pick[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bool take_leaf = leaf < n && (node >= made || hw[leaf] <= hw[node]);
        pick[c] = take_leaf ? leaf++ : node++;
      }
      hw[made] = hw[pick[0]] + hw[pick[1]];
      hpar[pick[0]] = (uint16_t)made;
      hpar[pick[1]] = (uint16_t)made;
      ++made;
    }
  }
  __syncthreads();
  // Each leaf's depth: the walk to the root (node 2n - 2) rises every step.
  if (t < n) {
    uint32_t depth = 1;
    if (n >= 2) {
      depth = 0;
      for (uint32_t j = t; j != 2u * n - 2u; j = hpar[j]) ++depth;
    }
    if (depth > kLmax) s.plan[5] = 1;
    leaf_len[t] = (uint8_t)(depth > kLmax ? kLmax : depth);
  }
  __syncthreads();
  if (s.plan[5]) {
    // Over-long codes were cut to kLmax; while the Kraft sum exceeds 1, the
    // longest code shorter than kLmax grows by one bit (ties: the lightest
    // leaf, i.e. the smallest count, then the largest exponent).
    if (t == 0) {
      uint32_t kraft = 0;
      for (uint32_t j = 0; j < n; ++j) kraft += 1u << (kLmax - leaf_len[j]);
      while (kraft > (1u << kLmax)) {
        uint32_t best = n, bl = 0;
        for (uint32_t j = 0; j < n; ++j) {
          const uint32_t l = leaf_len[j];
          if (l < kLmax && (best == n || l > bl)) { best = j; bl = l; }
        }
        kraft -= 1u << (kLmax - bl - 1u);
        leaf_len[best] = (uint8_t)(bl + 1u);
      }
    }
    __syncthreads();
  }
  if (t < n) s.len[sym_asc[t]] = leaf_len[t];
  __syncthreads();
  // Canonical codes: codes of one length are consecutive in exponent order,
  // and the first code of length L is (first of L-1 + count of L-1) << 1.
  const uint32_t l = owner ? s.len[t] : 0u;
  uint32_t rank = 0;
#pragma unroll
  for (uint32_t L = 1; L <= kLmax; ++L) {
    const uint64_t bm = __ballot(owner && l == L);
    if (l == L) rank = lanemask_lt_count(bm);
    if (owner && lane == 0) s.cbl[wave][L] = (uint32_t)__popcll(bm);
  }
  __syncthreads();
  if (owner) {
    uint32_t e = 0;
    if (l) {
      uint32_t code = 0, prev = 0;
      for (uint32_t L = 1; L <= l; ++L) {
        code = (code + prev) << 1;
        prev = s.cbl[0][L] + s.cbl[1][L] + s.cbl[2][L] + s.cbl[3][L];
      }
      for (uint32_t w = 0; w < wave; ++w) code += s.cbl[w][l];
      code += rank;
      e = (__builtin_bitreverse32(code) >> (32u - l)) | (l << 16);
    }
    s.enc[t] = e;
  }
  if (t < 128u) stage8(s)[16 + t] = (uint8_t)(s.len[2 * t] | (s.len[2 * t + 1] << 4));
  others();
  __syncthreads();
  return n;
}

__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kCW))) void hce_compress_kernel(
    const uint16_t* __restrict__ in, uint64_t n, uint8_t* __restrict__ out, uint64_t* __restrict__ out_bytes,
    CompressWs* __restrict__ ws, uint32_t nb, uint32_t spin_limit) {
  __shared__ HceEncSmem s;
  const uint32_t t = threadIdx.x, lane = t & 63u, seg = t >> 6;
  const uint32_t bid = blockIdx.x;
  const uint64_t first = (uint64_t)bid * kB;
  const uint32_t m = (uint32_t)((n - first) < kB ? (n - first) : kB);
  uint4 v[kPer];
  if (m == kB) {
    load_block_lanes(in + first, seg, lane, s, v);
  } else {
    load_lane_steps(in + first, m, seg, lane, v);
  }
  zero_hist(s);
  __syncthreads();
  uint32_t mode = 0, n_sym = 0, n_words = 0, rec_bytes = raw_bytes(m);
  uint32_t codes[16];   // step i's code bits (low 12) and length (high 4), two per word
  uint32_t cum_start = 0, base = 0;
  if (m == kB) {
    const uint32_t cnt = block_histogram<true>(v, s);
    __syncthreads();   // the sub-histograms are read: the staging buffer is free
    // the sign/fraction plane goes to the staging buffer while the code is built
    n_sym = build_code(cnt, s, [&] {
      uint8_t* sm = stage8(s) + kSmOff + 2048u * seg + lane;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t x = elem_of(v, i);
        sm[64u * i] = (uint8_t)(((x >> 8) & 0x80u) | (x & 0x7Fu));
      }
    });
    // First pass: this lane's bits in this segment.
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t w = word_of(v, k);
      const uint32_t e0 = s.enc[(w >> 7) & 0xFFu], e1 = s.enc[(w >> 23) & 0xFFu];
      const uint32_t c0 = (e0 & 0xFFFu) | ((e0 >> 16) << 12), c1 = (e1 & 0xFFFu) | ((e1 >> 16) << 12);
      codes[k] = c0 | (c1 << 16);
      bits += (e0 >> 16) + (e1 >> 16);
    }
    s.seg[seg][lane] = bits;
    __syncthreads();
    uint32_t total = 0;
#pragma unroll
    for (uint32_t q = 0; q < kSegs; ++q) {
      const uint32_t b = s.seg[q][lane];
      cum_start += q < seg ? b : 0u;
      total += b;
    }
    n_words = wave_sum((total + 31u) >> 5);        // every wave holds all 64 lanes
    base = wave_sum((cum_start + 31u) >> 5);       // words taken before this segment
    if (n_words <= kMaxWords) {
      mode = 2;
      rec_bytes = hce_coded_bytes(n_words);
    }
    __syncthreads();   // s.seg is read; it holds carried words from here on
  }
  if (t == 0) publish(&ws->desc[bid], (bid == 0 ? kFlagIncl : kFlagAgg) | rec_bytes);
  uint8_t* st8 = stage8(s);
  if (mode == 2) {   // the sign/fraction plane is in place (written while the code was built)
    uint32_t* words = stage32(s) + kWordsOff / 4;
    if (t < 3u && ((n_words + t) * 4u) < ((4u * n_words + 15u) & ~15u)) words[n_words + t] = 0;  // padding
    // Second pass: write this segment's codes of this lane.
    uint32_t cum = cum_start;
    const uint32_t w0 = cum >> 5;             // the word holding bit cum
    const bool carry_in = (cum & 31u) != 0;   // word w0 was taken and begun by the previous segment
    uint32_t r = (cum + 31u) >> 5;            // words of this lane taken so far
    uint32_t written = w0;                    // words of this lane finished (w0 counts when carried)
    uint64_t acc = 0;                         // bits from bit 32 * written on
    uint32_t pa = 0, pb = 0, pend = 0;        // words taken here and not yet written, oldest first
    uint32_t carry = 0, b = base;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t c = (codes[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const uint32_t l = c >> 12;
      const bool need = cum + l > 32u * r;
      const uint64_t mask = __ballot(need);
      if (need) {
        const uint32_t p = b + lanemask_lt_count(mask);
        if (pend == 0) pa = p; else pb = p;
        ++pend;
        ++r;
      }
      b += (uint32_t)__popcll(mask);
      acc |= (uint64_t)(c & 0xFFFu) << (cum - 32u * written);
      cum += l;
      if (cum >= 32u * (written + 1u)) {
        const uint32_t wv = (uint32_t)acc;
        if (carry_in && written == w0) {
          carry = wv;
        } else {
          words[pa] = wv;
          pa = pb;
          --pend;
        }
        acc >>= 32;
        ++written;
      }
    }
    uint32_t last = 0xFFFFu;
    if (cum > 32u * written) {   // an unfinished last word: the next segment adds its bits
      words[pa] = (uint32_t)acc;
      last = pa;
    }
    s.seg[seg][lane] = carry;
    s.lastpos[seg][lane] = (uint16_t)last;
    __syncthreads();
    if (carry_in) words[s.lastpos[seg - 1][lane]] |= s.seg[seg][lane];
    if (t == 0) {
      uint32_t* h = stage32(s);
      h[0] = 2u | (kLmax << 8) | (n_sym << 16);
      h[1] = m;
      h[2] = n_words;
      h[3] = rec_bytes;
    }
  } else {
    // raw record: the m words, then zero padding (elements past m loaded as 0)
    uint16_t* st16 = reinterpret_cast<uint16_t*>(st8 + 16);
    const uint32_t lim = (m + 7u) & ~7u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t idx = 2048u * seg + 64u * i + lane;
      if (idx < lim) st16[idx] = (uint16_t)elem_of(v, i);
    }
    if (t == 0) {
      uint32_t* h = stage32(s);
      h[0] = 0;
      h[1] = m;
      h[2] = 0;
      h[3] = rec_bytes;
    }
  }
  __syncthreads();
  if (t < 64) {
    bool ok = true;
    const uint64_t excl = lookback_wave(ws, bid, rec_bytes, spin_limit, &ok);
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
  copy_out(s, out + off, rec_bytes);
  if (t == 0) reinterpret_cast<uint64_t*>(out + 32)[bid] = off;
  if (bid == nb - 1 && t < 64) {   // the last block's first wave
    const bool failed = lookback_failed(ws, nb, spin_limit);
    if (t == 0) {
      const uint64_t tot = off + rec_bytes;
      write_stream_header(out, kHceMagic, kB, n, nb, tot);
      *out_bytes = failed ? 0 : tot;
    }
  }
}

// Decoding table entry: exponent << 7 | code length; every window that
// starts no code holds kNoCode (length field 15, above any real length).
// Two levels: the primary table is indexed by the top kPrimBits bits of the
// 12-bit window and resolves every code of at most kPrimBits bits.  Canonical
// codes put all longer codes after the shorter ones, so their windows form
// one range [T, kraft) that starts 4-aligned; a primary entry inside it holds
// kLongMark and (window - T) << 4, and the secondary table resolves the
// window.  Codes of 11 and 12 bits cover at most 2 windows each, so the
// secondary table needs at most 2 * 256 entries plus the rounding of kraft up
// to 4.  A block thus takes 4.1 KB of LDS instead of the 9.2 KB of one
// 4096-entry table, and more blocks stay resident per compute unit.  Both
// tables are stored at bit-reversed indices (lookup).
constexpr uint16_t kNoCode = 0xFFFFu;
constexpr uint32_t kPrimBits = 10;
constexpr uint32_t kLongMark = 14u;
constexpr uint32_t kSecMax = 2 * 256 + 4;

struct HceDecSmem {
  uint16_t lut[1u << kPrimBits];  // first 10 window bits (reversed) -> entry, or a pointer into lut2
  uint16_t lut2[kSecMax];         // windows T .. round_up(kraft, 4) - 1 (last 2 bits reversed) -> entry
  uint16_t start[257];            // window value where each code (in length, exponent order) begins
  uint16_t ent[256];              // table entry of each code in that order
};

// Entry of the code at the bottom of buf (the next stream bits, first bit in
// bit 0).  The tables are indexed by the window's bits in stream order from
// the low bit up, i.e. by the bit-reversed window (fill_table stores them so):
// the primary by stream bits 0..9, the secondary by its range offset plus
// stream bits 10 and 11.  A decoder that holds its bits this way adds a word
// with one shift and needs no bit reversal per word.
__device__ __forceinline__ uint32_t lookup(const HceDecSmem& s, uint64_t buf) {
  const uint32_t w = (uint32_t)buf;
  uint32_t e = s.lut[w & ((1u << kPrimBits) - 1u)];
  if ((e & 15u) == kLongMark) e = s.lut2[(e >> 4) | ((w >> kPrimBits) & ((1u << (kLmax - kPrimBits)) - 1u))];
  return e;
}

// Fills tbl[rev(i)] for i in [0, cnt) with the entry of the code holding
// window base + stride*i: kNoCode at or past kraft, a pointer into lut2 at
// or past long_from, else the code's own entry.  rev reverses the low
// rev_bits bits of i (the lookup indexes by stream bits, first bit lowest).  Lane l takes entries
// [per*l, per*l + per); it starts at a lane-dependent point of its run and
// wraps, so that the lanes' writes fall in different banks, and walks the
// codes forward (they are consecutive in window order).
__device__ __forceinline__ void fill_table(const HceDecSmem& s, uint16_t* tbl, uint32_t cnt, uint32_t per,
                                           uint32_t base, uint32_t stride, uint32_t long_from, uint32_t n_sym,
                                           uint32_t kraft, uint32_t rev_bits) {
  const uint32_t lane = threadIdx.x, i0 = per * lane;
  if (i0 >= cnt) return;
  const uint32_t len = (cnt - i0) < per ? (cnt - i0) : per, r = lane % len;
  uint32_t k0, k;
  {
    uint32_t lo = 0, hi = n_sym;   // the last code starting at or before the run's first window
    while (hi - lo > 1u) {
      const uint32_t mid = (lo + hi) >> 1;
      if (s.start[mid] <= base + stride * i0) lo = mid; else hi = mid;
    }
    k0 = lo;
    hi = n_sym;                    // ... at or before the window where this lane starts
    while (hi - lo > 1u) {
      const uint32_t mid = (lo + hi) >> 1;
      if (s.start[mid] <= base + stride * (i0 + r)) lo = mid; else hi = mid;
    }
    k = lo;
  }
  uint32_t next = s.start[k + 1], cur = s.ent[k];
  for (uint32_t j = 0; j < len; ++j) {
    uint32_t o = r + j;
    if (o >= len) o -= len;
    if (o == 0 && j != 0) { k = k0; next = s.start[k + 1]; cur = s.ent[k]; }
    const uint32_t x = base + stride * (i0 + o);
    while (x >= next && k + 1 < n_sym) { ++k; next = s.start[k + 1]; cur = s.ent[k]; }
    const uint32_t i = i0 + o, lowmask = (1u << rev_bits) - 1u;
    tbl[(i & ~lowmask) | (__builtin_bitreverse32(i & lowmask) >> (32u - rev_bits))] =
        x >= kraft ? kNoCode : x >= long_from ? (uint16_t)(((x - long_from) << 4) | kLongMark) : (uint16_t)cur;
  }
}

// One code per lane per step for the 256 steps, writing each element (the
// sign and fraction from the record's plane, the exponent decoded).  The
// words are read from the record through a window of 128 words held across
// the wave (lane k: word wbase + k, and wbase + 64 + k).  Returns this
// lane's "corrupt" flag.
__device__ __forceinline__ bool decode_steps(const HceDecSmem& s, const uint8_t* __restrict__ rec, uint32_t n_words,
                                             uint16_t* __restrict__ dst) {
  const uint32_t lane = threadIdx.x;
  const uint32_t* wg = reinterpret_cast<const uint32_t*>(rec + kWordsOff);
  // Window words are loaded without a condition: a lane whose word would lie
  // past the last one reads the record's first word instead (always in
  // bounds), a value that a valid stream never takes.  A select between the
  // loaded word and a constant would make the wave wait for the load at once
  // (and, counters being in order, for every load and store before it); as
  // it is, the first wait comes when the window is used, steps later.
  const uint32_t* hdr = reinterpret_cast<const uint32_t*>(rec);
  uint32_t win = *(lane < n_words ? wg + lane : hdr);
  uint32_t win2 = *(64u + lane < n_words ? wg + 64u + lane : hdr);
  uint32_t wbase = 0, base = 0, avail = 0;
  uint64_t buf = 0;   // the lane's next `avail` stream bits, from bit 0 up; zero above them
  bool bad = false;
  const uint8_t* smp = rec + kSmOff + lane;
  uint32_t smn[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) smn[q] = smp[64u * q];
  for (uint32_t i0 = 0; i0 < kSteps; i0 += 8) {
    uint32_t smv[8];   // sign at bit 15 (and 7), fraction in bits 0..6 (and 8..14)
#pragma unroll
    for (int q = 0; q < 8; ++q) smv[q] = smn[q] * 0x101u;
    if (i0 + 8 < kSteps) {
#pragma unroll
      for (int q = 0; q < 8; ++q) smn[q] = smp[64u * (i0 + 8 + q)];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t e = lookup(s, buf);
      uint32_t L = e & 15u;
      const bool need = L > avail;
      const uint64_t mask = __ballot(need);
      if (mask) {
        const uint32_t taken = (uint32_t)__popcll(mask);
        const uint32_t rel = base - wbase + lanemask_lt_count(mask);   // < 128: base - wbase < 64 at every step
        uint32_t word = __shfl(win, (int)(rel & 63u), 64);
        if (base - wbase + taken > 64u) {   // the last word taken here lies in the second window
          const uint32_t w2 = __shfl(win2, (int)(rel & 63u), 64);
          word = rel >= 64u ? w2 : word;
        }
        if (need) {
          buf |= (uint64_t)word << avail;
          avail += 32;
          e = lookup(s, buf);
          L = e & 15u;
        }
        base += taken;
        if (base - wbase >= 64u) {
          wbase += 64;
          win = win2;
          const uint32_t nx = wbase + 64u + lane;
          win2 = *(nx < n_words ? wg + nx : hdr);
        }
      }
      bad |= L == 15u;   // no code in the window: a corrupt stream
      buf >>= L;
      avail -= L;
      // sign and fraction from the plane, the exponent (bits 7..14) from the entry, whose bits 4..6 and 15 are zero
      uint32_t o;   // one bitfield insert (the compiler splits the plain form into an AND and an AND-OR)
      asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(o) : "s"(0x807Fu), "v"(smv[q]), "v"(e));
      dst[64u * (i0 + q) + lane] = (uint16_t)o;
    }
  }
  return bad || base != n_words || buf != 0;
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(8))) void hce_decompress_kernel(const uint8_t* __restrict__ in, uint64_t in_bytes,
                                                            uint16_t* __restrict__ out, uint64_t n,
                                                            int32_t* __restrict__ status, uint32_t nb) {
  __shared__ HceDecSmem s;
  const uint32_t lane = threadIdx.x, bid = blockIdx.x;
  const uint64_t first = (uint64_t)bid * kB;
  const uint32_t m = (uint32_t)((n - first) < kB ? (n - first) : kB);
  uint64_t off = 0;
  uint32_t len = 0;
  if (!check_stream(in, in_bytes, kHceMagic, n, nb, bid, &off, &len)) {
    if (lane == 0) atomicExch(status, (int32_t)HC_ERR_CORRUPT_STREAM);
    return;
  }
  const uint8_t* rec = in + off;
  const uint4 h = ld16(rec);
  const uint32_t mode = h.x & 0xFFu, lmax = (h.x >> 8) & 0xFFu, n_sym = h.x >> 16, n_words = h.z, rb = h.w;
  const bool hok = h.y == m && rb == len &&
                   ((mode == 0 && lmax == 0 && n_sym == 0 && n_words == 0 && rb == raw_bytes(m)) ||
                    (mode == 2 && m == kB && lmax == kLmax && n_sym >= 1 && n_sym <= 256 && n_words <= kMaxWords &&
                     rb == hce_coded_bytes(n_words)));
  if (!hok) {
    if (lane == 0) atomicExch(status, (int32_t)HC_ERR_CORRUPT_STREAM);
    return;
  }
  uint16_t* dst = out + first;
  bool bad = false;
  if (mode == 0) {
    const uint32_t chunks = (rb - 16u) / 16u;   // 8 elements each, padding zero
    for (uint32_t c = lane; c < chunks; c += 64) {
      const uint4 q = ld16(rec + 16 + 16 * c);
      if (8u * c + 8u <= m) {
        st16(dst + 8u * c, q);
      } else {
        const uint32_t wds[4] = {q.x, q.y, q.z, q.w};
        for (uint32_t k = 0; k < 8; ++k) {
          const uint32_t x = (wds[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
          if (8u * c + k < m) dst[8u * c + k] = (uint16_t)x;
          else bad |= x != 0;
        }
      }
    }
  } else {
    const uint32_t* wg = reinterpret_cast<const uint32_t*>(rec + kWordsOff);
    // Code lengths: lane holds exponents lane + 64 k.
    uint32_t ln[4];
    uint32_t kraft = 0, present = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t e = lane + 64u * k;
      const uint32_t byte = rec[16 + (e >> 1)];
      ln[k] = (e & 1u) ? (byte >> 4) : (byte & 0xFu);
      bad |= ln[k] > kLmax;
      kraft += (ln[k] && ln[k] <= kLmax) ? (1u << (kLmax - ln[k])) : 0u;
      present += ln[k] != 0;
    }
    kraft = wave_sum(kraft);
    present = wave_sum(present);
    bad |= kraft > (1u << kLmax) || present != n_sym;
    if (!__ballot(bad)) {
      // canonical tables (uniform): codes of each length, their first code and first sorted index
      uint32_t cnt[kLmax + 1], fcode[kLmax + 1], fidx[kLmax + 1], run[kLmax + 1];
      cnt[0] = 0;
#pragma unroll
      for (uint32_t L = 1; L <= kLmax; ++L) {
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) c += (uint32_t)__popcll(__ballot(ln[k] == L));
        cnt[L] = c;
      }
      uint32_t code = 0, idx = 0;
#pragma unroll
      for (uint32_t L = 1; L <= kLmax; ++L) {
        code = (code + cnt[L - 1]) << 1;
        fcode[L] = code;
        fidx[L] = idx;
        idx += cnt[L];
        run[L] = 0;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (uint32_t L = 1; L <= kLmax; ++L) {
          const uint64_t bm = __ballot(ln[k] == L);
          if (ln[k] == L) {
            const uint32_t r = run[L] + lanemask_lt_count(bm);
            s.ent[fidx[L] + r] = (uint16_t)(((lane + 64u * k) << 7) | L);
            s.start[fidx[L] + r] = (uint16_t)((fcode[L] + r) << (kLmax - L));
          }
          run[L] += (uint32_t)__popcll(bm);
        }
      }
      if (lane == 0) s.start[n_sym] = (uint16_t)kraft;   // end of the last code's range
      __syncthreads();
      // The two tables.  T: the windows of the codes of at most kPrimBits
      // bits, which come first; the secondary table covers T .. kraft
      // rounded up to 4.
      {
        uint32_t T = 0;
#pragma unroll
        for (uint32_t L = 1; L <= kPrimBits; ++L) T += cnt[L] << (kLmax - L);
        const uint32_t sec = ((kraft + 3u) & ~3u) - T;   // <= 2 * 256 + 3 (codes of 11, 12 bits)
        fill_table(s, s.lut, 1u << kPrimBits, (1u << kPrimBits) / 64u, 0u, 1u << (kLmax - kPrimBits), T, n_sym,
                   kraft, kPrimBits);
        fill_table(s, s.lut2, sec < kSecMax ? sec : kSecMax, (kSecMax + 63u) / 64u, T, 1u, 0xFFFFFFFFu, n_sym,
                   kraft, kLmax - kPrimBits);
      }
      __syncthreads();
      bad = decode_steps(s, rec, n_words, dst);
      // zero padding after the last word
      const uint32_t pw = n_words + lane;
      if (lane < 3u && 4u * pw < ((4u * n_words + 15u) & ~15u)) bad |= wg[pw] != 0;
    }
  }
  if (__ballot(bad) && lane == 0) atomicExch(status, (int32_t)HC_ERR_CORRUPT_STREAM);
}

}  // namespace

hipError_t launch_hce_compress(const uint16_t* in, size_t n, void* out, uint64_t* out_bytes, void* ws,
                               hipStream_t stream) {
  const size_t nb = ceil_div(n, kB);
  if (nb == 0) return launch_empty_stream(out, kHceMagic, out_bytes, stream);
  if (nb >= (1ull << 31)) return hipErrorInvalidValue;
  hipError_t e = launch_fill_u32(ws, 0u, compress_ws_bytes(n) / 4, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hce_compress_kernel, dim3((uint32_t)nb), dim3(kCT), 0, stream, in, (uint64_t)n,
                     static_cast<uint8_t*>(out), out_bytes, static_cast<CompressWs*>(ws), (uint32_t)nb,
                     lookback_spin_limit());
  return hipGetLastError();
}

hipError_t launch_hce_decompress(const void* in, size_t in_bytes, uint16_t* out, size_t n, int32_t* status,
                                 hipStream_t stream) {
  hipError_t e = launch_fill_u32(status, 0u, 1, stream);
  if (e != hipSuccess) return e;
  const size_t nb = ceil_div(n, kB);
  if (nb >= (1ull << 31)) return hipErrorInvalidValue;
  if (nb == 0) return launch_check_empty_stream(in, in_bytes, kHceMagic, status, stream);
  hipLaunchKernelGGL(hce_decompress_kernel, dim3((uint32_t)nb), dim3(64), 0, stream,
                     static_cast<const uint8_t*>(in), (uint64_t)in_bytes, out, (uint64_t)n, status, (uint32_t)nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_zero_if_corrupt(status, out, n, stream);
}

}  // namespace hc
