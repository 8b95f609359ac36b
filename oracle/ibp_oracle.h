/*
 * ibp_oracle.h -- plain single-threaded CPU oracle for Invariant Bit Packing.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it and shares no
 * code, table or helper with it.
 *
 * Sources.  "FR summary" below is the gist.science French technical summary
 * of arXiv 2605.30728 ("Résumé Technique : Réduire le goulot d'étranglement
 * de la mémoire GPU par la compression sans perte pour le ML"); "KO summary"
 * is its Korean counterpart ("Reducing the GPU Memory Bottleneck with
 * Lossless Compression for ML -- Extended").  Both describe one method in
 * three steps (section "Algorithme central" / "핵심 알고리즘"):
 *   1. preprocessing: Mask and Bitval from a batch of tensors and a
 *      threshold T;
 *   2. compression: per chunk, a match test against Bitval at the masked
 *      positions, removal of the matched invariant bits, and a participation
 *      bit per chunk;
 *   3. decompression: every chunk rebuilt by putting Bitval's bits back.
 * Section "Intégration au système" adds fixed-size slots of which only the
 * compressed prefix is read, and a GPU-resident bitmask of compressed
 * tensors.
 *
 * Bit conventions (the pages fix none; these readings are listed with the
 * rest in the design notes):
 *   - a tensor is a bit string; bit i is bit (i mod 8) of byte i/8
 *     (LSB first), which is bit (i mod 32) of little-endian 32-bit word i/32;
 *   - chunk c of a tensor is bits [c*W, c*W + W);
 *   - Mask and Bitval are M-bit strings (same bit order); bit j of chunk c
 *     uses Mask/Bitval bit (c*W + j) mod M, so M is the period of the
 *     metadata along the tensor (M = tensor bits: one flag per position of
 *     the tensor; M = W: one pattern shared by every chunk);
 *   - a record is: n participation bits (bit c = 1 when chunk c matched and
 *     lost its invariant bits), zero-padded to H = 32*ceil(n/32) bits,
 *     followed by every chunk's kept bits in chunk order, each chunk's bits
 *     in ascending position, then zero bits up to a multiple of 32;
 *   - a slot of L bytes holds the record when 4*ceil(R/32) < L (bitmask bit
 *     1), else the raw tensor (bitmask bit 0).
 *
 * Return codes: 0 ok, -1 invalid argument, -5 corrupt record, -6 id out of
 * range.
 */
#ifndef IBP_ORACLE_H
#define IBP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IBP_REF_OK 0
#define IBP_REF_ERR_INVALID (-1)
#define IBP_REF_ERR_CORRUPT (-5)
#define IBP_REF_ERR_RANGE (-6)

/* Step 1 (FR/KO summary, "Algorithme central", preprocessing).
 * sample: n_sample tensors of tensor_bits bits each, bit-contiguous.
 * Every M-bit block of the sample is one observation.  Position j is
 * invariant when at least K = ceil(T * n_obs) observations agree on it
 * (product and ceiling in IEEE double); Bitval holds the agreed value there
 * and 0 elsewhere.  mask/bitval: M bits each (ceil(M/8) bytes), written. */
int ibp_ref_build_metadata(uint64_t tensor_bits, uint32_t W, uint32_t M, double T,
                           const uint8_t* sample, uint64_t n_sample,
                           uint8_t* mask, uint8_t* bitval);

/* Step 2 for one tensor: writes the record (zero padded to a multiple of 32
 * bits) into rec, whose capacity must be at least ibp_ref_max_record_bits()
 * bits, and its exact length R (before padding) into *rec_bits. */
int ibp_ref_encode_record(uint64_t tensor_bits, uint32_t W, uint32_t M,
                          const uint8_t* mask, const uint8_t* bitval,
                          const uint8_t* x, uint8_t* rec, uint64_t rec_cap_bits,
                          uint64_t* rec_bits);

/* Worst-case record length in bits (every chunk verbatim), padded to 32. */
uint64_t ibp_ref_max_record_bits(uint64_t tensor_bits, uint32_t W);

/* Length R of the record that starts at rec, read from its header alone;
 * -5 when the header padding bits are not zero or the record would not fit
 * in rec_avail_bits. */
int ibp_ref_record_bits(uint64_t tensor_bits, uint32_t W, uint32_t M,
                        const uint8_t* mask, const uint8_t* rec,
                        uint64_t rec_avail_bits, uint64_t* rec_bits);

/* Step 3 for one record: rebuilds the tensor into x (tensor_bits bits). */
int ibp_ref_decode_record(uint64_t tensor_bits, uint32_t W, uint32_t M,
                          const uint8_t* mask, const uint8_t* bitval,
                          const uint8_t* rec, uint64_t rec_avail_bits, uint8_t* x);

/* Batches of the two calls above (tensor i at xs + i*x_stride bytes,
 * record i at recs + i*rec_stride bytes); used by exhaustive tests. */
int ibp_ref_encode_records(uint64_t tensor_bits, uint32_t W, uint32_t M,
                           const uint8_t* mask, const uint8_t* bitval,
                           const uint8_t* xs, uint64_t n, uint64_t x_stride,
                           uint8_t* recs, uint64_t rec_stride, uint64_t* rec_bits);
int ibp_ref_decode_records(uint64_t tensor_bits, uint32_t W, uint32_t M,
                           const uint8_t* mask, const uint8_t* bitval,
                           const uint8_t* recs, uint64_t rec_stride, uint64_t n,
                           uint8_t* xs, uint64_t x_stride);

/* Slots ("Intégration au système"): n_tensors tensors of L bytes from src
 * into n_tensors slots of L bytes.  bitmask: ceil(n/32) words, fully
 * rewritten (bits past n are 0).  stored (nullable): bytes each slot holds.
 * Slot bytes after a record are written as zero. */
int ibp_ref_compress(uint64_t L, uint32_t W, uint32_t M,
                     const uint8_t* mask, const uint8_t* bitval,
                     const uint8_t* src, uint64_t n_tensors,
                     uint8_t* slots, uint32_t* bitmask, uint64_t* stored);

int ibp_ref_decompress(uint64_t L, uint32_t W, uint32_t M,
                       const uint8_t* mask, const uint8_t* bitval,
                       const uint8_t* slots, const uint32_t* bitmask,
                       uint64_t n_tensors, uint8_t* dst);

/* dst row i = tensor ids[i]; ids must lie in [0, n_slots). */
int ibp_ref_gather_decompress(uint64_t L, uint32_t W, uint32_t M,
                              const uint8_t* mask, const uint8_t* bitval,
                              const uint8_t* slots, uint64_t n_slots,
                              const uint32_t* bitmask, const int64_t* ids,
                              uint64_t n_ids, uint8_t* dst);

/* Packed cache (FR/KO summary, "Intégration au système": in the GPU
 * software cache of GNN frameworks, compressing the cached tensors raises
 * how many of them fit).  Item t is what slot t of ibp_ref_compress holds --
 * the record (4*ceil(R/32) bytes) when that is shorter than L, else the raw
 * tensor (L bytes) -- and the items are stored back to back: item t starts at
 * byte offsets[t], offsets[0] = 0 and offsets[t+1] = offsets[t] + the item's
 * bytes rounded up to a multiple of 16.  offsets has n_tensors + 1 entries.
 * Bytes between an item's end and the next offset are written as zero. */
int ibp_ref_packed_offsets(uint64_t L, uint32_t W, uint32_t M,
                           const uint8_t* mask, const uint8_t* bitval,
                           const uint8_t* src, uint64_t n_tensors, uint64_t* offsets);

/* Writes offsets, the items into buf and the bitmask (as ibp_ref_compress).
 * -6 when offsets[n_tensors] > capacity bytes; buf is then left untouched. */
int ibp_ref_compress_packed(uint64_t L, uint32_t W, uint32_t M,
                            const uint8_t* mask, const uint8_t* bitval,
                            const uint8_t* src, uint64_t n_tensors,
                            uint8_t* buf, uint64_t capacity, uint64_t* offsets,
                            uint32_t* bitmask);

/* dst row i = tensor ids[i] from a packed buffer of n_items items.  Item t
 * spans bytes [offsets[t], offsets[t+1]); a compressed item whose header
 * implies a record longer than that, or not shorter than L, is corrupt (-5),
 * and so is a raw item shorter than L.  ids outside [0, n_items): -6. */
int ibp_ref_gather_decompress_packed(uint64_t L, uint32_t W, uint32_t M,
                                     const uint8_t* mask, const uint8_t* bitval,
                                     const uint8_t* buf, const uint64_t* offsets,
                                     uint64_t n_items, const uint32_t* bitmask,
                                     const int64_t* ids, uint64_t n_ids, uint8_t* dst);

/* Headers in GPU memory ("Intégration au système" keeps the bitmask of
 * compressed slots in GPU memory; this layout keeps each compressed tensor's
 * header words there as well, so that what crosses the host link is payload
 * only).  Same compressed/raw decision as ibp_ref_compress.  For a compressed
 * tensor, slot t holds the record's payload words (record words hw .. end,
 * hw = ceil(n/32)) followed by zeros, and headers[t*hw .. t*hw+hw) holds its
 * header words; for a raw tensor the slot holds the tensor and its header
 * words are zero.  stored (nullable): payload bytes, or L when raw. */
int ibp_ref_compress_split(uint64_t L, uint32_t W, uint32_t M,
                           const uint8_t* mask, const uint8_t* bitval,
                           const uint8_t* src, uint64_t n_tensors,
                           uint8_t* slots, uint32_t* headers, uint32_t* bitmask, uint64_t* stored);

/* dst row i = tensor ids[i] from that layout (ids in [0, n_slots), else -6).
 * A compressed tensor whose header padding bits are set, or whose header
 * implies 4*ceil(R/32) >= L, is corrupt (-5). */
int ibp_ref_gather_decompress_split(uint64_t L, uint32_t W, uint32_t M,
                                    const uint8_t* mask, const uint8_t* bitval,
                                    const uint8_t* slots, uint64_t n_slots, const uint32_t* headers,
                                    const uint32_t* bitmask, const int64_t* ids, uint64_t n_ids,
                                    uint8_t* dst);

#ifdef __cplusplus
}
#endif
#endif
