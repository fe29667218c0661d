/*
 * hce_oracle.c -- CPU oracle of "HCE1", the entropy-coded exponent variant of
 * the lossless bf16 codec.
 *
 * TEST INFRASTRUCTURE ONLY, under the same rules as hc_oracle.c: only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark use it,
 * and it shares no code, header or table with the HIP library.
 *
 * Source: "CCCL: In-GPU Compression-Coupled Collective Communication",
 * section 4.1 (the 8-bit bf16 exponent is coded from a frequency table, sign
 * and fraction travel raw) and section 6.5 (the fixed-length CCCL core is
 * compared with an entropy coder, DietGPU, whose output is smaller by under
 * 7%).  This variant keeps everything of the fixed-length format except the
 * exponent code, which becomes a per-block Huffman code (Huffman's minimum
 * redundancy construction), written in canonical form (the code assignment
 * of RFC 1951, section 3.2.2) with lengths limited to 12 bits.
 *
 * Format HCE1 (little-endian; every padding byte and bit is zero):
 *  - stream: 32-byte header {u32 magic 0x31454348, u32 16384, u64 n,
 *    u32 n_blocks, u32 0, u64 total_bytes}; u64 rec_off[n_blocks] padded to
 *    16 bytes; the records in block order (as HCZ1, with its own magic).
 *  - record header (16 bytes): {u8 mode (0 raw, 2 coded), u8 lmax (12 coded,
 *    0 raw), u16 n_sym (coded: exponents present; raw 0), u32 m, u32 n_words
 *    (coded; raw 0), u32 rec_bytes}.
 *  - raw record: the m words, padded to 16 bytes.
 *  - coded record (m = 16384 only):
 *      [16, 144)     code length of exponent e (0 absent, 1..12) in the low
 *                    nibble of byte 16 + e/2 for even e, the high nibble for
 *                    odd e;
 *      [144, 16528)  sign/fraction plane, sm[i] = sign << 7 | fraction;
 *      [16528, ...)  the n_words 32-bit words of the lanes' streams,
 *                    interleaved as below, padded to 16 bytes.
 *    rec_bytes = 16528 + round_up(4 * n_words, 16).  A full block is coded
 *    when that is below the raw 16 + 32768 bytes, else raw; a partial tail
 *    block is raw.
 *  - lanes: the block is read by 64 lanes of 256 elements; lane j takes the
 *    elements 64 i + j, step i = 0..255 being its i-th.
 *  - a lane's bit stream is its 256 codes in step order, each code's most
 *    significant bit first; stream bit b is bit b mod 32 of the lane's word
 *    b / 32 (bits after the last code are zero).
 *  - word order: a decoder running the 64 lanes in lockstep over the steps
 *    takes a lane's next word when the bits it holds do not contain the
 *    lane's next code, lanes in increasing order within a step.  So word w
 *    of a lane is taken at the first step i whose code ends past bit 32 w of
 *    the lane's stream (the bits of codes 0..i exceed 32 w), and the words
 *    are stored in (that step, lane) order.  No per-lane offsets are
 *    stored; each lane pads only its own last word.
 *
 * Readings where the pages are silent (all this variant's own choices):
 *  - ties in the Huffman construction: leaves enter in increasing count,
 *    equal counts by decreasing exponent; when the next leaf and the next
 *    merged node weigh the same, the leaf is taken first.
 *  - a block with a single exponent codes it with length 1.
 *  - length limit 12 (a 4096-entry decoding table): lengths above 12 become
 *    12; then, while the Kraft sum exceeds 1, the longest code shorter than
 *    12 (ties: smallest count, then largest exponent) is made one bit longer.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { HCE_OK = 0, HCE_CORRUPT = 4 };

#define HCE_MAGIC 0x31454348u
#define HCE_B 16384u
#define HCE_LMAX 12
#define HCE_LANES 64
#define HCE_STEPS 256
#define HCE_SM_OFF 144u
#define HCE_WORDS_OFF 16528u

static size_t hce_ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }
static size_t hce_round_up(size_t a, size_t b) { return hce_ceil_div(a, b) * b; }
static void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void wr32(uint8_t *p, uint32_t v) { for (int k = 0; k < 4; ++k) p[k] = (uint8_t)(v >> (8 * k)); }
static void wr64(uint8_t *p, uint64_t v) { for (int k = 0; k < 8; ++k) p[k] = (uint8_t)(v >> (8 * k)); }
static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t rd32(const uint8_t *p) { uint32_t v = 0; for (int k = 3; k >= 0; --k) v = (v << 8) | p[k]; return v; }
static uint64_t rd64(const uint8_t *p) { uint64_t v = 0; for (int k = 7; k >= 0; --k) v = (v << 8) | p[k]; return v; }

static size_t hce_header_bytes(size_t nb) { return 32 + hce_round_up(8 * nb, 16); }
static size_t hce_raw_bytes(size_t m) { return 16 + hce_round_up(2 * m, 16); }
static size_t hce_coded_bytes(size_t n_words) { return HCE_WORDS_OFF + hce_round_up(4 * n_words, 16); }

/* Element index of lane j's step i inside a block. */
static size_t lane_elem(int j, int i) { return (size_t)HCE_LANES * (size_t)i + (size_t)j; }

/* ------------------------------------------------------------------------ */
/* Huffman code lengths                                                      */
/* ------------------------------------------------------------------------ */

static const uint32_t *g_cnt;   /* comparator context (single-threaded) */
static int by_count_up_exponent_down(const void *pa, const void *pb)
{
    int a = *(const int *)pa, b = *(const int *)pb;
    if (g_cnt[a] != g_cnt[b]) return g_cnt[a] < g_cnt[b] ? -1 : 1;
    return b - a;
}

/*
 * Code lengths of a minimum-redundancy (Huffman) code for the exponents with
 * a nonzero count, limited to lmax bits by the rule in the header.  The
 * construction takes the two lightest of (next leaf, next merged node) each
 * time; leaves are visited in increasing weight and merged nodes are made in
 * increasing weight, so the two fronts are always the lightest candidates.
 * len[256] receives the lengths (0 for absent exponents).  Returns n_sym.
 */
int or_huff_lengths(const uint32_t *cnt, int lmax, uint8_t *len)
{
    int sym[256], n = 0;
    memset(len, 0, 256);
    for (int e = 0; e < 256; ++e)
        if (cnt[e]) sym[n++] = e;
    if (n == 0) return 0;
    if (n == 1) { len[sym[0]] = 1; return 1; }
    g_cnt = cnt;
    qsort(sym, (size_t)n, sizeof(int), by_count_up_exponent_down);
    uint64_t w[511];
    int parent[511];
    for (int i = 0; i < n; ++i) w[i] = cnt[sym[i]];
    int leaf = 0, node = n, made = n;
    for (int k = 0; k < n - 1; ++k) {
        int pick[2];
        for (int c = 0; c < 2; ++c) {
            if (leaf < n && (node >= made || w[leaf] <= w[node])) pick[c] = leaf++;
            else pick[c] = node++;
        }
        w[made] = w[pick[0]] + w[pick[1]];
        parent[pick[0]] = made;
        parent[pick[1]] = made;
        ++made;
    }
    const int root = 2 * n - 2;
    int depth[256];
    int deepest = 0;
    for (int i = 0; i < n; ++i) {
        int d = 0;
        for (int j = i; j != root; j = parent[j]) ++d;
        depth[i] = d;
        if (d > deepest) deepest = d;
    }
    for (int i = 0; i < n; ++i) len[sym[i]] = (uint8_t)(depth[i] > lmax ? lmax : depth[i]);
    if (deepest > lmax) {
        uint64_t kraft = 0, cap = (uint64_t)1 << lmax;
        for (int i = 0; i < n; ++i) kraft += (uint64_t)1 << (lmax - len[sym[i]]);
        while (kraft > cap) {
            int best = -1;
            for (int e = 0; e < 256; ++e) {
                if (!cnt[e] || len[e] >= lmax) continue;
                if (best < 0 || len[e] > len[best] ||
                    (len[e] == len[best] && (cnt[e] < cnt[best] || (cnt[e] == cnt[best] && e > best))))
                    best = e;
            }
            kraft -= (uint64_t)1 << (lmax - len[best] - 1);
            len[best]++;
        }
    }
    return n;
}

/*
 * Canonical codes from lengths (RFC 1951, section 3.2.2): count the codes of
 * each length, the first code of length l is (first code of l-1 + count of
 * l-1) << 1, and codes of one length go to the symbols in increasing order.
 * code[256] receives each present symbol's code (right-aligned).
 */
void or_huff_codes(const uint8_t *len, int lmax, uint32_t *code)
{
    uint32_t bl_count[33] = {0}, next_code[33] = {0};
    for (int e = 0; e < 256; ++e) if (len[e]) bl_count[len[e]]++;
    uint32_t c = 0;
    bl_count[0] = 0;
    for (int bits = 1; bits <= lmax; ++bits) {
        c = (c + bl_count[bits - 1]) << 1;
        next_code[bits] = c;
    }
    for (int e = 0; e < 256; ++e) code[e] = len[e] ? next_code[len[e]]++ : 0;
}

/* ------------------------------------------------------------------------ */
/* Encoder                                                                   */
/* ------------------------------------------------------------------------ */

size_t or_hce_bound(size_t n)
{
    size_t nb = hce_ceil_div(n, HCE_B), total = hce_header_bytes(nb);
    for (size_t k = 0; k < nb; ++k) total += hce_raw_bytes(k + 1 < nb ? HCE_B : n - k * HCE_B);
    return total;
}

/* A lane's stream as bits, and when each of its words is first needed. */
typedef struct {
    uint8_t bit[HCE_STEPS * HCE_LMAX];
    int nbits;
    int need_step[HCE_STEPS * HCE_LMAX / 32];   /* per word */
    int nwords;
} lane_stream_t;

static void build_lane(const uint16_t *blk, int t, const uint8_t *len, const uint32_t *code, lane_stream_t *ls)
{
    int cum = 0;
    ls->nwords = 0;
    for (int i = 0; i < HCE_STEPS; ++i) {
        uint32_t e = (blk[lane_elem(t, i)] >> 7) & 0xFF;
        int l = len[e];
        for (int b = l - 1; b >= 0; --b) ls->bit[cum++] = (uint8_t)((code[e] >> b) & 1u);
        /* every word whose first bit this code reaches is needed at step i */
        while (32 * ls->nwords < cum) ls->need_step[ls->nwords++] = i;
    }
    ls->nbits = cum;
}

static uint32_t lane_word(const lane_stream_t *ls, int w)
{
    uint32_t v = 0;
    for (int j = 0; j < 32; ++j) {
        int b = 32 * w + j;
        if (b < ls->nbits && ls->bit[b]) v |= 1u << j;
    }
    return v;
}

typedef struct { int mode; uint32_t n_sym, n_words, rec_bytes; } hce_plan_t;

/* Plans and (when out != NULL) writes one block's record. */
static hce_plan_t hce_block(const uint16_t *blk, size_t m, uint8_t *out)
{
    hce_plan_t p = {0, 0, 0, (uint32_t)hce_raw_bytes(m)};
    uint8_t len[256];
    uint32_t code[256];
    static lane_stream_t lanes[HCE_LANES];
    if (m == HCE_B) {
        uint32_t cnt[256] = {0};
        for (size_t i = 0; i < m; ++i) cnt[(blk[i] >> 7) & 0xFF]++;
        p.n_sym = (uint32_t)or_huff_lengths(cnt, HCE_LMAX, len);
        or_huff_codes(len, HCE_LMAX, code);
        uint32_t words = 0;
        for (int t = 0; t < HCE_LANES; ++t) {
            build_lane(blk, t, len, code, &lanes[t]);
            words += (uint32_t)lanes[t].nwords;
        }
        size_t coded = hce_coded_bytes(words);
        if (coded < hce_raw_bytes(m)) {
            p.mode = 2;
            p.n_words = words;
            p.rec_bytes = (uint32_t)coded;
        }
    }
    if (p.mode != 2) p.n_sym = 0;
    if (!out) return p;
    memset(out, 0, p.rec_bytes);
    out[0] = (uint8_t)p.mode;
    out[1] = (uint8_t)(p.mode == 2 ? HCE_LMAX : 0);
    wr16(out + 2, (uint16_t)p.n_sym);
    wr32(out + 4, (uint32_t)m);
    wr32(out + 8, p.n_words);
    wr32(out + 12, p.rec_bytes);
    if (p.mode == 0) {
        for (size_t i = 0; i < m; ++i) wr16(out + 16 + 2 * i, blk[i]);
        return p;
    }
    for (int e = 0; e < 256; ++e) out[16 + e / 2] |= (uint8_t)(len[e] << (4 * (e & 1)));
    for (size_t i = 0; i < m; ++i) out[HCE_SM_OFF + i] = (uint8_t)(((blk[i] >> 8) & 0x80) | (blk[i] & 0x7F));
    /* the words in (need step, lane) order */
    size_t pos = 0;
    int next_word[HCE_LANES] = {0};
    for (int step = 0; step < HCE_STEPS; ++step)
        for (int l = 0; l < HCE_LANES; ++l) {
            const lane_stream_t *ls = &lanes[l];
            if (next_word[l] < ls->nwords && ls->need_step[next_word[l]] == step) {
                wr32(out + HCE_WORDS_OFF + 4 * pos, lane_word(ls, next_word[l]));
                ++pos;
                ++next_word[l];
            }
        }
    return p;
}

/*
 * Compress n bf16 words into an HCE1 stream.  Returns the stream size, or 0
 * when cap is below or_hce_bound(n).
 */
size_t or_hce_compress(const uint16_t *in, size_t n, uint8_t *out, size_t cap)
{
    size_t nb = hce_ceil_div(n, HCE_B), hdr = hce_header_bytes(nb);
    if (cap < or_hce_bound(n)) return 0;
    memset(out, 0, hdr);
    wr32(out + 0, HCE_MAGIC);
    wr32(out + 4, HCE_B);
    wr64(out + 8, (uint64_t)n);
    wr32(out + 16, (uint32_t)nb);
    wr32(out + 20, 0);
    size_t off = hdr;
    for (size_t k = 0; k < nb; ++k) {
        size_t m = (k + 1) * HCE_B <= n ? HCE_B : n - k * HCE_B;
        wr64(out + 32 + 8 * k, (uint64_t)off);
        hce_plan_t p = hce_block(in + k * HCE_B, m, out + off);
        off += p.rec_bytes;
    }
    wr64(out + 24, (uint64_t)off);
    return off;
}

/* One block's plan (mode, n_sym, n_words, rec_bytes) for the tests. */
int or_hce_plan_block(const uint16_t *v, size_t m, uint32_t *plan4)
{
    if (m == 0 || m > HCE_B) return 1;
    hce_plan_t p = hce_block(v, m, NULL);
    plan4[0] = (uint32_t)p.mode;
    plan4[1] = p.n_sym;
    plan4[2] = p.n_words;
    plan4[3] = p.rec_bytes;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Decoder                                                                   */
/* ------------------------------------------------------------------------ */

/* Canonical decoding tables from the lengths: for each length l the first
 * code, the count and the index of its first symbol in (length, exponent)
 * order. */
typedef struct {
    uint32_t first_code[HCE_LMAX + 1], count[HCE_LMAX + 1], first_idx[HCE_LMAX + 1];
    uint8_t sorted[256];
} canon_t;

static void canon_tables(const uint8_t *len, canon_t *c)
{
    memset(c, 0, sizeof *c);
    for (int e = 0; e < 256; ++e) if (len[e]) c->count[len[e]]++;
    uint32_t code = 0, idx = 0;
    for (int l = 1; l <= HCE_LMAX; ++l) {
        code = (code + c->count[l - 1]) << 1;
        c->first_code[l] = code;
        c->first_idx[l] = idx;
        idx += c->count[l];
    }
    uint32_t fill[HCE_LMAX + 1];
    memcpy(fill, c->first_idx, sizeof fill);
    for (int e = 0; e < 256; ++e) if (len[e]) c->sorted[fill[len[e]]++] = (uint8_t)e;
}

/* Decode one code from the `avail` low bits of buf (stream order = bit 0
 * first).  Returns the code length and the symbol, 0 when the available
 * bits hold no whole code, -1 when no code of up to lmax bits matches. */
static int decode_one(uint64_t buf, int avail, const canon_t *c, int *sym)
{
    uint32_t code = 0;
    for (int l = 1; l <= HCE_LMAX; ++l) {
        if (l > avail) return 0;
        code = (code << 1) | (uint32_t)((buf >> (l - 1)) & 1u);
        if (code - c->first_code[l] < c->count[l]) {   /* unsigned: code >= first_code too */
            *sym = c->sorted[c->first_idx[l] + code - c->first_code[l]];
            return l;
        }
    }
    return -1;
}

static int decode_coded(const uint8_t *rec, uint32_t rb, uint16_t *dst)
{
    uint32_t n_sym = rd16(rec + 2), n_words = rd32(rec + 8);
    if (rec[1] != HCE_LMAX || n_sym < 1 || rb != hce_coded_bytes(n_words)) return 0;
    uint8_t len[256];
    uint32_t present = 0;
    uint64_t kraft = 0;
    for (int e = 0; e < 256; ++e) {
        len[e] = (uint8_t)((rec[16 + e / 2] >> (4 * (e & 1))) & 0xF);
        if (len[e] > HCE_LMAX) return 0;
        if (len[e]) { present++; kraft += (uint64_t)1 << (HCE_LMAX - len[e]); }
    }
    if (present != n_sym || kraft > ((uint64_t)1 << HCE_LMAX)) return 0;
    canon_t c;
    canon_tables(len, &c);
    const uint8_t *words = rec + HCE_WORDS_OFF;
    uint64_t buf[HCE_LANES] = {0};
    int avail[HCE_LANES] = {0};
    uint32_t pos = 0;
    for (int i = 0; i < HCE_STEPS; ++i) {
        for (int l = 0; l < HCE_LANES; ++l) {
            int sym = 0, got = decode_one(buf[l], avail[l], &c, &sym);
            if (got == 0) {          /* take the next word */
                if (pos >= n_words) return 0;
                buf[l] |= (uint64_t)rd32(words + 4 * pos) << avail[l];
                avail[l] += 32;
                ++pos;
                got = decode_one(buf[l], avail[l], &c, &sym);
            }
            if (got <= 0) return 0;
            buf[l] >>= got;
            avail[l] -= got;
            size_t idx = lane_elem(l, i);
            uint8_t sm = rec[HCE_SM_OFF + idx];
            dst[idx] = (uint16_t)(((uint32_t)(sm & 0x80) << 8) | ((uint32_t)sym << 7) | (sm & 0x7F));
        }
    }
    if (pos != n_words) return 0;
    for (int l = 0; l < HCE_LANES; ++l) if (buf[l]) return 0;   /* padding bits are zero */
    for (size_t b = HCE_WORDS_OFF + 4 * (size_t)n_words; b < rb; ++b) if (rec[b]) return 0;
    return 1;
}

/*
 * Decompress an HCE1 stream of in_bytes bytes holding n elements.  Every
 * field is checked before use (magic, sizes, offsets, lengths table with
 * Kraft sum <= 1, word counts, every code decodable, every word used, zero
 * padding); a corrupt stream returns 4 and leaves out zero.
 */
int or_hce_decompress(const uint8_t *in, size_t in_bytes, uint16_t *out, size_t n)
{
    memset(out, 0, n * 2);
    size_t nb = hce_ceil_div(n, HCE_B), hdr = hce_header_bytes(nb);
    if (in_bytes < hdr) return HCE_CORRUPT;
    if (rd32(in) != HCE_MAGIC || rd32(in + 4) != HCE_B || rd64(in + 8) != n || rd32(in + 16) != nb ||
        rd32(in + 20) != 0)
        return HCE_CORRUPT;
    uint64_t total = rd64(in + 24);
    if (total > in_bytes || total < hdr) return HCE_CORRUPT;
    for (size_t i = 32 + 8 * nb; i < hdr; ++i) if (in[i]) return HCE_CORRUPT;
    uint64_t expect = hdr;
    for (size_t k = 0; k < nb; ++k) {
        uint64_t off = rd64(in + 32 + 8 * k);
        if (off != expect || off + 16 > total) goto corrupt;
        const uint8_t *rec = in + off;
        size_t m = (k + 1) * HCE_B <= n ? HCE_B : n - k * HCE_B;
        uint32_t mode = rec[0], rb = rd32(rec + 12);
        if (rd32(rec + 4) != m || off + rb > total) goto corrupt;
        uint16_t *dst = out + k * HCE_B;
        if (mode == 0) {
            if (rec[1] != 0 || rd16(rec + 2) != 0 || rd32(rec + 8) != 0 || rb != hce_raw_bytes(m)) goto corrupt;
            for (size_t i = 0; i < m; ++i) dst[i] = rd16(rec + 16 + 2 * i);
            for (size_t i = 16 + 2 * m; i < rb; ++i) if (rec[i]) goto corrupt;
        } else if (mode == 2) {
            if (m != HCE_B || !decode_coded(rec, rb, dst)) goto corrupt;
        } else {
            goto corrupt;
        }
        expect = off + rb;
    }
    if (expect != total) goto corrupt;
    return HCE_OK;
corrupt:
    memset(out, 0, n * 2);
    return HCE_CORRUPT;
}
