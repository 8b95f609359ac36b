/*
 * oracle_sanitize_driver.c -- runs every entry point of the C oracle on
 * seeded random formats and data, including corrupt records and ids out of
 * range, with every buffer allocated at exactly the size the call needs.
 * tests/test_oracle_sanitized.py builds it together with oracle/ibp_oracle.c
 * under gcc's AddressSanitizer and UndefinedBehaviorSanitizer: an access
 * past a buffer, a use of freed memory or undefined arithmetic aborts it.
 * Test infrastructure only.  Exit status 0 when every round trip is exact
 * and every error case returns its documented code.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/ibp_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void) { /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}

static uint32_t below(uint32_t n) { return (uint32_t)(next_u64() % n); }

static int bit_get(const uint8_t* a, uint64_t i) { return (a[i >> 3] >> (i & 7)) & 1; }

static void bit_put(uint8_t* a, uint64_t i, int v) {
    if (v)
        a[i >> 3] |= (uint8_t)(1u << (i & 7));
    else
        a[i >> 3] &= (uint8_t)~(1u << (i & 7));
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int failures = 0;

#define EXPECT(cond, ...)                       \
    do {                                        \
        if (!(cond)) {                          \
            fprintf(stderr, __VA_ARGS__);       \
            fputc('\n', stderr);                \
            ++failures;                         \
        }                                       \
    } while (0)

/* One format: W-bit chunks, an M-bit period, tensors of L bytes. */
static void run_format(uint32_t W, uint32_t M, uint64_t L, uint32_t n, int density_pct, int match_pct) {
    const uint64_t tb = 8 * L;
    const uint64_t n_chunks = tb / W;
    const size_t mbytes = (M + 7) / 8;
    uint8_t* mask = xmalloc(mbytes);
    uint8_t* bitval = xmalloc(mbytes);
    memset(mask, 0, mbytes);
    memset(bitval, 0, mbytes);
    for (uint32_t j = 0; j < M; ++j) {
        const int m = (int)below(100) < density_pct;
        bit_put(mask, j, m);
        bit_put(bitval, j, m && below(2));
    }
    /* tensors: random bits, then each chunk made to match with match_pct % */
    uint8_t* src = xmalloc((size_t)(n * L));
    for (uint64_t i = 0; i < n * L; ++i) src[i] = (uint8_t)next_u64();
    for (uint32_t t = 0; t < n; ++t) {
        uint8_t* x = src + t * L;
        for (uint64_t c = 0; c < n_chunks; ++c) {
            if ((int)below(100) >= match_pct) continue;
            for (uint32_t b = 0; b < W; ++b) {
                const uint64_t j = (c * W + b) % M;
                if (bit_get(mask, j)) bit_put(x, c * W + b, bit_get(bitval, j));
            }
        }
    }

    /* metadata from the tensors themselves (only exercised, not compared) */
    {
        uint8_t* m2 = xmalloc(mbytes);
        uint8_t* b2 = xmalloc(mbytes);
        EXPECT(ibp_ref_build_metadata(tb, W, M, 0.9, src, n, m2, b2) == IBP_REF_OK, "build_metadata W=%u M=%u", W, M);
        free(m2);
        free(b2);
    }

    /* single records */
    const uint64_t cap = ibp_ref_max_record_bits(tb, W);
    uint8_t* rec = xmalloc((size_t)(cap / 8));
    uint8_t* back = xmalloc((size_t)L);
    for (uint32_t t = 0; t < n; ++t) {
        uint64_t R = 0, R2 = 0;
        EXPECT(ibp_ref_encode_record(tb, W, M, mask, bitval, src + t * L, rec, cap, &R) == IBP_REF_OK,
               "encode_record W=%u", W);
        EXPECT(ibp_ref_record_bits(tb, W, M, mask, rec, cap, &R2) == IBP_REF_OK && R2 == R, "record_bits W=%u", W);
        const uint64_t avail = 32 * ((R + 31) / 32);
        EXPECT(ibp_ref_decode_record(tb, W, M, mask, bitval, rec, avail, back) == IBP_REF_OK &&
                   memcmp(back, src + t * L, (size_t)L) == 0,
               "decode_record W=%u t=%u", W, t);
        /* one 32-bit word short of the record: corrupt, never a read past it */
        if (avail >= 64) {
            uint8_t* cut = xmalloc((size_t)((avail - 32) / 8));
            memcpy(cut, rec, (size_t)((avail - 32) / 8));
            EXPECT(ibp_ref_decode_record(tb, W, M, mask, bitval, cut, avail - 32, back) == IBP_REF_ERR_CORRUPT,
                   "short record W=%u", W);
            free(cut);
        }
    }

    /* slots, bitmask, decompress, gather */
    const uint32_t bw = (n + 31) / 32;
    uint8_t* slots = xmalloc((size_t)(n * L));
    uint32_t* bm = xmalloc(4 * (size_t)bw);
    uint64_t* stored = xmalloc(8 * (size_t)n);
    uint8_t* dst = xmalloc((size_t)(n * L));
    EXPECT(ibp_ref_compress(L, W, M, mask, bitval, src, n, slots, bm, stored) == IBP_REF_OK, "compress W=%u", W);
    EXPECT(ibp_ref_decompress(L, W, M, mask, bitval, slots, bm, n, dst) == IBP_REF_OK &&
               memcmp(dst, src, (size_t)(n * L)) == 0,
           "decompress W=%u M=%u L=%llu", W, M, (unsigned long long)L);
    const uint32_t n_ids = 2 * n + 1;
    int64_t* ids = xmalloc(8 * (size_t)n_ids);
    for (uint32_t i = 0; i < n_ids; ++i) ids[i] = below(n);
    uint8_t* gdst = xmalloc((size_t)(n_ids * L));
    EXPECT(ibp_ref_gather_decompress(L, W, M, mask, bitval, slots, n, bm, ids, n_ids, gdst) == IBP_REF_OK,
           "gather W=%u", W);
    for (uint32_t i = 0; i < n_ids; ++i)
        EXPECT(memcmp(gdst + i * L, src + ids[i] * L, (size_t)L) == 0, "gather row %u W=%u", i, W);
    ids[n_ids - 1] = n; /* out of range */
    EXPECT(ibp_ref_gather_decompress(L, W, M, mask, bitval, slots, n, bm, ids, n_ids, gdst) == IBP_REF_ERR_RANGE,
           "gather range W=%u", W);
    ids[n_ids - 1] = 0;
    /* a compressed slot with its header padding bits set: corrupt */
    const uint64_t hw = (n_chunks + 31) / 32;
    for (uint32_t t = 0; t < n; ++t) {
        if (!((bm[t >> 5] >> (t & 31)) & 1) || (n_chunks % 32) == 0) continue;
        uint8_t* bad = xmalloc((size_t)L);
        memcpy(bad, slots + t * L, (size_t)L);
        bit_put(bad, 32 * (hw - 1) + 31, 1);
        uint32_t one = 1;
        EXPECT(ibp_ref_decompress(L, W, M, mask, bitval, bad, &one, 1, back) == IBP_REF_ERR_CORRUPT,
               "header padding W=%u", W);
        free(bad);
        break;
    }

    /* packed cache */
    uint64_t* off = xmalloc(8 * ((size_t)n + 1));
    EXPECT(ibp_ref_packed_offsets(L, W, M, mask, bitval, src, n, off) == IBP_REF_OK, "packed_offsets W=%u", W);
    const uint64_t total = off[n];
    uint8_t* buf = xmalloc((size_t)total);
    uint64_t* off2 = xmalloc(8 * ((size_t)n + 1));
    uint32_t* bm2 = xmalloc(4 * (size_t)bw);
    EXPECT(ibp_ref_compress_packed(L, W, M, mask, bitval, src, n, buf, total, off2, bm2) == IBP_REF_OK &&
               memcmp(off, off2, 8 * ((size_t)n + 1)) == 0,
           "compress_packed W=%u", W);
    if (total >= 16)
        EXPECT(ibp_ref_compress_packed(L, W, M, mask, bitval, src, n, buf, total - 16, off2, bm2) ==
                   IBP_REF_ERR_RANGE,
               "packed capacity W=%u", W);
    EXPECT(ibp_ref_gather_decompress_packed(L, W, M, mask, bitval, buf, off, n, bm, ids, n_ids, gdst) == IBP_REF_OK,
           "gather_packed W=%u", W);
    for (uint32_t i = 0; i < n_ids; ++i)
        EXPECT(memcmp(gdst + i * L, src + ids[i] * L, (size_t)L) == 0, "packed row %u W=%u", i, W);
    if (n >= 2) { /* an item cut to 16 bytes or misaligned: corrupt (or range), never a read outside */
        uint64_t* bad = xmalloc(8 * ((size_t)n + 1));
        memcpy(bad, off, 8 * ((size_t)n + 1));
        bad[1] = bad[0] + 16;
        int64_t id0 = 0;
        const int r = ibp_ref_gather_decompress_packed(L, W, M, mask, bitval, buf, bad, n, bm, &id0, 1, gdst);
        EXPECT(r == IBP_REF_OK || r == IBP_REF_ERR_CORRUPT, "packed cut W=%u: %d", W, r);
        memcpy(bad, off, 8 * ((size_t)n + 1));
        bad[1] += 4;
        const int r2 = ibp_ref_gather_decompress_packed(L, W, M, mask, bitval, buf, bad, n, bm, &id0, 1, gdst);
        EXPECT(r2 == IBP_REF_OK || r2 == IBP_REF_ERR_CORRUPT, "packed misaligned W=%u: %d", W, r2);
        free(bad);
    }

    /* headers in GPU memory */
    uint8_t* sslots = xmalloc((size_t)(n * L));
    uint32_t* headers = xmalloc(4 * (size_t)(n * hw));
    uint32_t* bm3 = xmalloc(4 * (size_t)bw);
    uint64_t* st3 = xmalloc(8 * (size_t)n);
    EXPECT(ibp_ref_compress_split(L, W, M, mask, bitval, src, n, sslots, headers, bm3, st3) == IBP_REF_OK,
           "compress_split W=%u", W);
    EXPECT(ibp_ref_gather_decompress_split(L, W, M, mask, bitval, sslots, n, headers, bm3, ids, n_ids, gdst) ==
               IBP_REF_OK,
           "gather_split W=%u", W);
    for (uint32_t i = 0; i < n_ids; ++i)
        EXPECT(memcmp(gdst + i * L, src + ids[i] * L, (size_t)L) == 0, "split row %u W=%u", i, W);

    free(st3);
    free(bm3);
    free(headers);
    free(sslots);
    free(bm2);
    free(off2);
    free(buf);
    free(off);
    free(gdst);
    free(ids);
    free(dst);
    free(stored);
    free(bm);
    free(slots);
    free(back);
    free(rec);
    free(src);
    free(bitval);
    free(mask);
}

int main(void) {
    static const uint32_t widths[] = {1, 2, 3, 5, 7, 8, 32, 64, 128, 256, 512, 1024};
    int formats = 0;
    for (int round = 0; round < 120; ++round) {
        const uint32_t W = widths[below(sizeof(widths) / sizeof(widths[0]))];
        /* L: a multiple of 4 bytes holding a whole number of chunks */
        uint64_t n_chunks = 1 + below(W >= 256 ? 24 : 160);
        uint64_t L = n_chunks * W / 8;
        while ((n_chunks * W) % 32 != 0 || L % 4 != 0 || L == 0) {
            ++n_chunks;
            L = n_chunks * W / 8;
        }
        /* M: W times a divisor of the chunk count */
        uint64_t d = 1 + below((uint32_t)n_chunks);
        while (n_chunks % d) --d;
        const uint32_t M = (uint32_t)(d * W);
        const uint32_t n = 1 + below(40);
        const int density = (int)below(101);
        const int match = (int)below(101);
        run_format(W, M, L, n, density, match);
        ++formats;
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle sanitized run: %d formats ok\n", formats);
    return 0;
}
