/*
 * ibp_oracle.c -- plain, bit-at-a-time CPU oracle for Invariant Bit Packing.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline of the
 * benchmark).  Shares nothing with the HIP library.  Conventions, sources and
 * return codes are documented in ibp_oracle.h.  Every loop below walks single
 * bits in the order the method states them; nothing is blocked, fused or
 * reordered, so each function can be checked against the description by eye.
 */
#include "ibp_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int get_bit(const uint8_t* buf, uint64_t i) {
    return (buf[i >> 3] >> (i & 7)) & 1;
}

static void put_bit(uint8_t* buf, uint64_t i, int v) {
    uint8_t m = (uint8_t)(1u << (i & 7));
    if (v)
        buf[i >> 3] |= m;
    else
        buf[i >> 3] &= (uint8_t)~m;
}

static uint64_t header_bits(uint64_t n_chunks) { return 32 * ((n_chunks + 31) / 32); }

static uint64_t round_up32(uint64_t bits) { return 32 * ((bits + 31) / 32); }

/* Shape rules: chunks tile the tensor, the metadata period is a whole number
 * of chunks and tiles the tensor. */
static int geometry_ok(uint64_t tensor_bits, uint32_t W, uint32_t M) {
    if (W == 0 || M == 0 || tensor_bits == 0) return 0;
    if (M % W != 0) return 0;
    if (tensor_bits % W != 0) return 0;
    if (tensor_bits % M != 0) return 0;
    return 1;
}

/* ------------------------------------------------------------------ */
/* Step 1: preprocessing (FR/KO summary, "Algorithme central" step 1).  */
/* ------------------------------------------------------------------ */
int ibp_ref_build_metadata(uint64_t tensor_bits, uint32_t W, uint32_t M, double T,
                           const uint8_t* sample, uint64_t n_sample,
                           uint8_t* mask, uint8_t* bitval) {
    if (!geometry_ok(tensor_bits, W, M)) return IBP_REF_ERR_INVALID;
    if (!(T > 0.5 && T <= 1.0)) return IBP_REF_ERR_INVALID;
    if (!sample || !mask || !bitval || n_sample == 0) return IBP_REF_ERR_INVALID;

    uint64_t n_obs = n_sample * (tensor_bits / M);
    uint64_t* ones = (uint64_t*)calloc(M, sizeof(uint64_t));
    if (!ones) return IBP_REF_ERR_INVALID;

    /* Count, for every position j of the period, how many observations
     * hold a 1 there. */
    for (uint64_t obs = 0; obs < n_obs; ++obs)
        for (uint32_t j = 0; j < M; ++j) ones[j] += (uint64_t)get_bit(sample, obs * M + j);

    /* Threshold: a position is invariant when at least K observations
     * agree, K = ceil(T * n_obs) computed in IEEE double. */
    double prod = T * (double)n_obs;
    uint64_t K = (uint64_t)ceil(prod);

    for (uint32_t j = 0; j < M; ++j) {
        uint64_t c1 = ones[j];
        uint64_t c0 = n_obs - c1;
        uint64_t agree = c1 > c0 ? c1 : c0;
        int invariant = agree >= K;
        put_bit(mask, j, invariant);
        put_bit(bitval, j, invariant && c1 > c0);
    }
    free(ones);
    return IBP_REF_OK;
}

/* ------------------------------------------------------------------ */
/* Step 2: compression of one tensor into a record.                     */
/* ------------------------------------------------------------------ */
uint64_t ibp_ref_max_record_bits(uint64_t tensor_bits, uint32_t W) {
    if (W == 0) return 0;
    return round_up32(header_bits(tensor_bits / W) + tensor_bits);
}

/* Match test of chunk c: every masked position holds Bitval's value. */
static int chunk_matches(uint32_t W, uint32_t M, const uint8_t* mask, const uint8_t* bitval,
                         const uint8_t* x, uint64_t c) {
    for (uint32_t b = 0; b < W; ++b) {
        uint64_t i = c * W + b;
        uint64_t j = i % M;
        if (get_bit(mask, j) && get_bit(x, i) != get_bit(bitval, j)) return 0;
    }
    return 1;
}

int ibp_ref_encode_record(uint64_t tensor_bits, uint32_t W, uint32_t M,
                          const uint8_t* mask, const uint8_t* bitval,
                          const uint8_t* x, uint8_t* rec, uint64_t rec_cap_bits,
                          uint64_t* rec_bits) {
    if (!geometry_ok(tensor_bits, W, M)) return IBP_REF_ERR_INVALID;
    if (!mask || !bitval || !x || !rec || !rec_bits) return IBP_REF_ERR_INVALID;
    uint64_t cap_needed = ibp_ref_max_record_bits(tensor_bits, W);
    if (rec_cap_bits < cap_needed) return IBP_REF_ERR_INVALID;

    uint64_t n = tensor_bits / W;
    uint64_t H = header_bits(n);
    memset(rec, 0, (size_t)(cap_needed / 8));

    /* Participation bits: bit c of the header is 1 when chunk c matched. */
    for (uint64_t c = 0; c < n; ++c) put_bit(rec, c, chunk_matches(W, M, mask, bitval, x, c));

    /* Payload: a matched chunk keeps only its non-invariant bits (in
     * ascending position, closing the gaps); an unmatched chunk is copied
     * verbatim. */
    uint64_t pos = H;
    for (uint64_t c = 0; c < n; ++c) {
        int p = get_bit(rec, c);
        for (uint32_t b = 0; b < W; ++b) {
            uint64_t i = c * W + b;
            uint64_t j = i % M;
            if (!p || !get_bit(mask, j)) put_bit(rec, pos++, get_bit(x, i));
        }
    }
    *rec_bits = pos; /* bits [pos, round_up32(pos)) stay zero */
    return IBP_REF_OK;
}

/* ------------------------------------------------------------------ */
/* Step 3: decompression of one record.                                 */
/* ------------------------------------------------------------------ */
int ibp_ref_record_bits(uint64_t tensor_bits, uint32_t W, uint32_t M,
                        const uint8_t* mask, const uint8_t* rec,
                        uint64_t rec_avail_bits, uint64_t* rec_bits) {
    if (!geometry_ok(tensor_bits, W, M)) return IBP_REF_ERR_INVALID;
    if (!mask || !rec || !rec_bits) return IBP_REF_ERR_INVALID;
    uint64_t n = tensor_bits / W;
    uint64_t H = header_bits(n);
    if (rec_avail_bits < H) return IBP_REF_ERR_CORRUPT;
    for (uint64_t c = n; c < H; ++c)
        if (get_bit(rec, c)) return IBP_REF_ERR_CORRUPT;

    /* Walk the chunks: a matched chunk holds W minus its masked bits, an
     * unmatched one holds W bits. */
    uint64_t R = H;
    for (uint64_t c = 0; c < n; ++c) {
        int p = get_bit(rec, c);
        for (uint32_t b = 0; b < W; ++b) {
            uint64_t j = (c * W + b) % M;
            if (!p || !get_bit(mask, j)) R += 1;
        }
    }
    if (R > rec_avail_bits) return IBP_REF_ERR_CORRUPT;
    *rec_bits = R;
    return IBP_REF_OK;
}

int ibp_ref_decode_record(uint64_t tensor_bits, uint32_t W, uint32_t M,
                          const uint8_t* mask, const uint8_t* bitval,
                          const uint8_t* rec, uint64_t rec_avail_bits, uint8_t* x) {
    uint64_t R;
    int st = ibp_ref_record_bits(tensor_bits, W, M, mask, rec, rec_avail_bits, &R);
    if (st != IBP_REF_OK) return st;
    if (!bitval || !x) return IBP_REF_ERR_INVALID;

    uint64_t n = tensor_bits / W;
    uint64_t pos = header_bits(n);
    /* Rebuild: at a masked position of a matched chunk the bit comes from
     * Bitval, everywhere else it is the next stored bit. */
    for (uint64_t c = 0; c < n; ++c) {
        int p = get_bit(rec, c);
        for (uint32_t b = 0; b < W; ++b) {
            uint64_t i = c * W + b;
            uint64_t j = i % M;
            int bit;
            if (p && get_bit(mask, j))
                bit = get_bit(bitval, j);
            else
                bit = get_bit(rec, pos++);
            put_bit(x, i, bit);
        }
    }
    return IBP_REF_OK;
}

int ibp_ref_encode_records(uint64_t tensor_bits, uint32_t W, uint32_t M,
                           const uint8_t* mask, const uint8_t* bitval,
                           const uint8_t* xs, uint64_t n, uint64_t x_stride,
                           uint8_t* recs, uint64_t rec_stride, uint64_t* rec_bits) {
    uint64_t need = ibp_ref_max_record_bits(tensor_bits, W);
    if (rec_stride * 8 < need) return IBP_REF_ERR_INVALID;
    for (uint64_t i = 0; i < n; ++i) {
        int st = ibp_ref_encode_record(tensor_bits, W, M, mask, bitval, xs + i * x_stride,
                                       recs + i * rec_stride, rec_stride * 8, &rec_bits[i]);
        if (st != IBP_REF_OK) return st;
    }
    return IBP_REF_OK;
}

int ibp_ref_decode_records(uint64_t tensor_bits, uint32_t W, uint32_t M,
                           const uint8_t* mask, const uint8_t* bitval,
                           const uint8_t* recs, uint64_t rec_stride, uint64_t n,
                           uint8_t* xs, uint64_t x_stride) {
    for (uint64_t i = 0; i < n; ++i) {
        int st = ibp_ref_decode_record(tensor_bits, W, M, mask, bitval, recs + i * rec_stride,
                                       rec_stride * 8, xs + i * x_stride);
        if (st != IBP_REF_OK) return st;
    }
    return IBP_REF_OK;
}

/* ------------------------------------------------------------------ */
/* Fixed-size slots and the bitmask ("Intégration au système").         */
/* ------------------------------------------------------------------ */
static void set_mask_bit(uint32_t* bitmask, uint64_t t, int v) {
    uint32_t m = 1u << (t % 32);
    if (v)
        bitmask[t / 32] |= m;
    else
        bitmask[t / 32] &= ~m;
}

static int mask_bit(const uint32_t* bitmask, uint64_t t) { return (bitmask[t / 32] >> (t % 32)) & 1; }

int ibp_ref_compress(uint64_t L, uint32_t W, uint32_t M,
                     const uint8_t* mask, const uint8_t* bitval,
                     const uint8_t* src, uint64_t n_tensors,
                     uint8_t* slots, uint32_t* bitmask, uint64_t* stored) {
    uint64_t tbits = 8 * L;
    if (!geometry_ok(tbits, W, M)) return IBP_REF_ERR_INVALID;
    if (!src || !slots || !bitmask) return IBP_REF_ERR_INVALID;
    uint64_t cap = ibp_ref_max_record_bits(tbits, W);
    uint8_t* rec = (uint8_t*)malloc((size_t)(cap / 8));
    if (!rec) return IBP_REF_ERR_INVALID;
    memset(bitmask, 0, (size_t)(4 * ((n_tensors + 31) / 32)));

    for (uint64_t t = 0; t < n_tensors; ++t) {
        const uint8_t* x = src + t * L;
        uint8_t* slot = slots + t * L;
        uint64_t R;
        int st = ibp_ref_encode_record(tbits, W, M, mask, bitval, x, rec, cap, &R);
        if (st != IBP_REF_OK) {
            free(rec);
            return st;
        }
        uint64_t words = (R + 31) / 32;
        if (4 * words < L) {
            /* compressed: the slot holds the record, the tail is unused */
            memset(slot, 0, (size_t)L);
            memcpy(slot, rec, (size_t)(4 * words));
            set_mask_bit(bitmask, t, 1);
            if (stored) stored[t] = 4 * words;
        } else {
            /* no saving: the slot holds the tensor as it is */
            memcpy(slot, x, (size_t)L);
            set_mask_bit(bitmask, t, 0);
            if (stored) stored[t] = L;
        }
    }
    free(rec);
    return IBP_REF_OK;
}

/* Decode one slot; a compressed slot whose record would not be strictly
 * shorter than the slot is corrupt (the compressor never writes one). */
static int decode_slot(uint64_t L, uint32_t W, uint32_t M, const uint8_t* mask,
                       const uint8_t* bitval, const uint8_t* slot, int compressed, uint8_t* out) {
    if (!compressed) {
        memcpy(out, slot, (size_t)L);
        return IBP_REF_OK;
    }
    uint64_t R;
    int st = ibp_ref_record_bits(8 * L, W, M, mask, slot, 8 * L, &R);
    if (st != IBP_REF_OK) return st;
    if (4 * ((R + 31) / 32) >= L) return IBP_REF_ERR_CORRUPT;
    return ibp_ref_decode_record(8 * L, W, M, mask, bitval, slot, 8 * L, out);
}

int ibp_ref_decompress(uint64_t L, uint32_t W, uint32_t M,
                       const uint8_t* mask, const uint8_t* bitval,
                       const uint8_t* slots, const uint32_t* bitmask,
                       uint64_t n_tensors, uint8_t* dst) {
    if (!geometry_ok(8 * L, W, M)) return IBP_REF_ERR_INVALID;
    if (!slots || !bitmask || !dst) return IBP_REF_ERR_INVALID;
    for (uint64_t t = 0; t < n_tensors; ++t) {
        int st = decode_slot(L, W, M, mask, bitval, slots + t * L, mask_bit(bitmask, t), dst + t * L);
        if (st != IBP_REF_OK) return st;
    }
    return IBP_REF_OK;
}

int ibp_ref_gather_decompress(uint64_t L, uint32_t W, uint32_t M,
                              const uint8_t* mask, const uint8_t* bitval,
                              const uint8_t* slots, uint64_t n_slots,
                              const uint32_t* bitmask, const int64_t* ids,
                              uint64_t n_ids, uint8_t* dst) {
    if (!geometry_ok(8 * L, W, M)) return IBP_REF_ERR_INVALID;
    if (!slots || !bitmask || !ids || !dst) return IBP_REF_ERR_INVALID;
    for (uint64_t i = 0; i < n_ids; ++i) {
        int64_t id = ids[i];
        if (id < 0 || (uint64_t)id >= n_slots) return IBP_REF_ERR_RANGE;
        int st = decode_slot(L, W, M, mask, bitval, slots + (uint64_t)id * L,
                             mask_bit(bitmask, (uint64_t)id), dst + i * L);
        if (st != IBP_REF_OK) return st;
    }
    return IBP_REF_OK;
}

/* ---------------------------------------------------------------------------
 * Packed cache: the slot items of ibp_ref_compress stored back to back.
 * ------------------------------------------------------------------------- */

/* Bytes item t takes: its record when that is shorter than L, else L. */
static int item_bytes(uint64_t L, uint32_t W, uint32_t M, const uint8_t* mask, const uint8_t* bitval,
                      const uint8_t* x, uint8_t* rec, uint64_t cap, uint64_t* bytes, int* compressed) {
    uint64_t R;
    int st = ibp_ref_encode_record(8 * L, W, M, mask, bitval, x, rec, cap, &R);
    if (st != IBP_REF_OK) return st;
    uint64_t words = (R + 31) / 32;
    *compressed = 4 * words < L;
    *bytes = *compressed ? 4 * words : L;
    return IBP_REF_OK;
}

static uint64_t round16(uint64_t b) { return (b + 15) / 16 * 16; }

int ibp_ref_packed_offsets(uint64_t L, uint32_t W, uint32_t M,
                           const uint8_t* mask, const uint8_t* bitval,
                           const uint8_t* src, uint64_t n_tensors, uint64_t* offsets) {
    if (!geometry_ok(8 * L, W, M)) return IBP_REF_ERR_INVALID;
    if (!offsets || (n_tensors && !src)) return IBP_REF_ERR_INVALID;
    uint64_t cap = ibp_ref_max_record_bits(8 * L, W);
    uint8_t* rec = (uint8_t*)malloc((size_t)(cap / 8));
    if (!rec) return IBP_REF_ERR_INVALID;
    offsets[0] = 0;
    for (uint64_t t = 0; t < n_tensors; ++t) {
        uint64_t bytes;
        int comp;
        int st = item_bytes(L, W, M, mask, bitval, src + t * L, rec, cap, &bytes, &comp);
        if (st != IBP_REF_OK) {
            free(rec);
            return st;
        }
        offsets[t + 1] = offsets[t] + round16(bytes);
    }
    free(rec);
    return IBP_REF_OK;
}

int ibp_ref_compress_packed(uint64_t L, uint32_t W, uint32_t M,
                            const uint8_t* mask, const uint8_t* bitval,
                            const uint8_t* src, uint64_t n_tensors,
                            uint8_t* buf, uint64_t capacity, uint64_t* offsets,
                            uint32_t* bitmask) {
    int st = ibp_ref_packed_offsets(L, W, M, mask, bitval, src, n_tensors, offsets);
    if (st != IBP_REF_OK) return st;
    if (offsets[n_tensors] > capacity) return IBP_REF_ERR_RANGE;
    if (!bitmask || (capacity && !buf)) return IBP_REF_ERR_INVALID;
    uint64_t cap = ibp_ref_max_record_bits(8 * L, W);
    uint8_t* rec = (uint8_t*)malloc((size_t)(cap / 8));
    if (!rec) return IBP_REF_ERR_INVALID;
    memset(bitmask, 0, (size_t)(4 * ((n_tensors + 31) / 32)));
    for (uint64_t t = 0; t < n_tensors; ++t) {
        const uint8_t* x = src + t * L;
        uint8_t* item = buf + offsets[t];
        uint64_t bytes;
        int comp;
        st = item_bytes(L, W, M, mask, bitval, x, rec, cap, &bytes, &comp);
        if (st != IBP_REF_OK) {
            free(rec);
            return st;
        }
        memset(item, 0, (size_t)(offsets[t + 1] - offsets[t]));
        memcpy(item, comp ? rec : x, (size_t)bytes);
        set_mask_bit(bitmask, t, comp);
    }
    free(rec);
    return IBP_REF_OK;
}

int ibp_ref_gather_decompress_packed(uint64_t L, uint32_t W, uint32_t M,
                                     const uint8_t* mask, const uint8_t* bitval,
                                     const uint8_t* buf, const uint64_t* offsets,
                                     uint64_t n_items, const uint32_t* bitmask,
                                     const int64_t* ids, uint64_t n_ids, uint8_t* dst) {
    if (!geometry_ok(8 * L, W, M)) return IBP_REF_ERR_INVALID;
    if (!offsets || !bitmask || (n_ids && (!buf || !ids || !dst))) return IBP_REF_ERR_INVALID;
    for (uint64_t i = 0; i < n_ids; ++i) {
        int64_t id = ids[i];
        if (id < 0 || (uint64_t)id >= n_items) return IBP_REF_ERR_RANGE;
        uint64_t a = offsets[id], b = offsets[id + 1];
        if (b < a) return IBP_REF_ERR_CORRUPT;
        const uint8_t* item = buf + a;
        uint8_t* out = dst + i * L;
        if (!mask_bit(bitmask, (uint64_t)id)) {
            if (b - a < L) return IBP_REF_ERR_CORRUPT;
            memcpy(out, item, (size_t)L);
            continue;
        }
        uint64_t R;
        int st = ibp_ref_record_bits(8 * L, W, M, mask, item, 8 * (b - a), &R);
        if (st != IBP_REF_OK) return st;
        if (4 * ((R + 31) / 32) >= L) return IBP_REF_ERR_CORRUPT;
        st = ibp_ref_decode_record(8 * L, W, M, mask, bitval, item, 8 * (b - a), out);
        if (st != IBP_REF_OK) return st;
    }
    return IBP_REF_OK;
}

/* ---------------------------------------------------------------------------
 * Headers in GPU memory: the slot keeps the payload, the header words go to a
 * separate array.
 * ------------------------------------------------------------------------- */

int ibp_ref_compress_split(uint64_t L, uint32_t W, uint32_t M,
                           const uint8_t* mask, const uint8_t* bitval,
                           const uint8_t* src, uint64_t n_tensors,
                           uint8_t* slots, uint32_t* headers, uint32_t* bitmask, uint64_t* stored) {
    uint64_t tbits = 8 * L;
    if (!geometry_ok(tbits, W, M)) return IBP_REF_ERR_INVALID;
    if (n_tensors && (!src || !slots || !headers || !bitmask)) return IBP_REF_ERR_INVALID;
    uint64_t hw = ((tbits / W) + 31) / 32; /* header words */
    uint64_t cap = ibp_ref_max_record_bits(tbits, W);
    uint8_t* rec = (uint8_t*)malloc((size_t)(cap / 8));
    if (!rec) return IBP_REF_ERR_INVALID;
    memset(bitmask, 0, (size_t)(4 * ((n_tensors + 31) / 32)));
    for (uint64_t t = 0; t < n_tensors; ++t) {
        const uint8_t* x = src + t * L;
        uint8_t* slot = slots + t * L;
        uint32_t* hdr = headers + t * hw;
        uint64_t R;
        int st = ibp_ref_encode_record(tbits, W, M, mask, bitval, x, rec, cap, &R);
        if (st != IBP_REF_OK) {
            free(rec);
            return st;
        }
        uint64_t words = (R + 31) / 32;
        if (4 * words < L) {
            memcpy(hdr, rec, (size_t)(4 * hw));
            memset(slot, 0, (size_t)L);
            memcpy(slot, rec + 4 * hw, (size_t)(4 * (words - hw)));
            set_mask_bit(bitmask, t, 1);
            if (stored) stored[t] = 4 * (words - hw);
        } else {
            memset(hdr, 0, (size_t)(4 * hw));
            memcpy(slot, x, (size_t)L);
            set_mask_bit(bitmask, t, 0);
            if (stored) stored[t] = L;
        }
    }
    free(rec);
    return IBP_REF_OK;
}

int ibp_ref_gather_decompress_split(uint64_t L, uint32_t W, uint32_t M,
                                    const uint8_t* mask, const uint8_t* bitval,
                                    const uint8_t* slots, uint64_t n_slots, const uint32_t* headers,
                                    const uint32_t* bitmask, const int64_t* ids, uint64_t n_ids,
                                    uint8_t* dst) {
    uint64_t tbits = 8 * L;
    if (!geometry_ok(tbits, W, M)) return IBP_REF_ERR_INVALID;
    if (n_ids && (!slots || !headers || !bitmask || !ids || !dst)) return IBP_REF_ERR_INVALID;
    uint64_t hw = ((tbits / W) + 31) / 32;
    /* the record rebuilt in front of the decoder: header words, then the
     * whole slot (the header tells how much of it is payload) */
    uint8_t* rec = (uint8_t*)malloc((size_t)(4 * hw + L));
    if (!rec) return IBP_REF_ERR_INVALID;
    for (uint64_t i = 0; i < n_ids; ++i) {
        int64_t id = ids[i];
        if (id < 0 || (uint64_t)id >= n_slots) {
            free(rec);
            return IBP_REF_ERR_RANGE;
        }
        const uint8_t* slot = slots + (uint64_t)id * L;
        uint8_t* out = dst + i * L;
        if (!mask_bit(bitmask, (uint64_t)id)) {
            memcpy(out, slot, (size_t)L);
            continue;
        }
        memcpy(rec, headers + (uint64_t)id * hw, (size_t)(4 * hw));
        memcpy(rec + 4 * hw, slot, (size_t)L);
        uint64_t R;
        int st = ibp_ref_record_bits(tbits, W, M, mask, rec, 8 * (4 * hw + L), &R);
        if (st == IBP_REF_OK && 4 * ((R + 31) / 32) >= L) st = IBP_REF_ERR_CORRUPT;
        if (st == IBP_REF_OK) st = ibp_ref_decode_record(tbits, W, M, mask, bitval, rec, 8 * (4 * hw + L), out);
        if (st != IBP_REF_OK) {
            free(rec);
            return st;
        }
    }
    free(rec);
    return IBP_REF_OK;
}
