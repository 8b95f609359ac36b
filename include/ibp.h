/*
 * ibp.h -- C ABI of libibp, an MI355X (gfx950) implementation of Invariant
 * Bit Packing (IBP), a lossless codec for ML tensors.
 *
 * Sources cited below:
 *   FR summary = gist.science French technical summary of arXiv 2605.30728,
 *     "Résumé Technique : Réduire le goulot d'étranglement de la mémoire GPU
 *     par la compression sans perte pour le ML";
 *   KO summary = its Korean counterpart, "Reducing the GPU Memory
 *     Bottleneck with Lossless Compression for ML -- Extended".
 * Both describe the method in section "Algorithme central" / "핵심 알고리즘"
 * (1 preprocessing, 2 compression, 3 decompression) and its use in section
 * "Intégration au système" / "시스템 통합" (fixed-size slots, GPU bitmask).
 *
 * Format (the pages fix no bit layout; this is the layout every call uses):
 *   - a tensor of L bytes is a bit string, bit i = bit (i mod 32) of
 *     little-endian 32-bit word i/32; chunk c = bits [c*W, c*W + W);
 *   - Mask/Bitval are M-bit strings (M/32 words, same bit order); chunk c
 *     is tested against their bits (c*W .. c*W+W-1) mod M;
 *   - a record = n = 8L/W participation bits (1 = the chunk matched and lost
 *     its masked bits), zero padded to H = 32*ceil(n/32) bits, then each
 *     chunk's kept bits in chunk order and ascending bit position, then zero
 *     bits up to a multiple of 32 (R bits before padding);
 *   - slot t (L bytes at slots + t*L) holds the record when
 *     4*ceil(R/32) < L and bitmask bit t is 1; otherwise the slot holds the
 *     tensor unchanged and the bit is 0.  Bitmask bit t is bit t%32 of word
 *     t/32.  Slot bytes after a record are unspecified.
 *
 * Memory kinds.  "device" = hipMalloc'd memory of the handle's GPU.
 * "device or pinned" = device memory or page-locked host memory
 * (hipHostMalloc / torch pin_memory), which kernels read or write directly
 * over the host link (zero copy).  Pageable host memory is rejected with
 * IBP_ERR_INVALID_ARG.  The caller owns and frees every buffer passed in;
 * the library owns only what an ibp_meta_t holds.
 *
 * Calls are asynchronous on `stream` unless stated; argument checks happen
 * on the host before any launch and leave outputs untouched on error.  Errors
 * found by kernels (an id out of range, a corrupt record) are latched in the
 * handle and reported by ibp_check().  Calls on one handle may run on
 * different streams at once; calls on the same stream run in order, also
 * when several host threads issue them.
 *
 * Tensors longer than one tile (more than 8 KiB) are cut into tiles whose
 * start bits need per-stream scratch of the handle: an encode of a source in
 * pinned host memory, and a decode of records read over the host link, find
 * them by a decoupled look-back; an encode of a 16-byte aligned source in
 * device memory computes them first from the source (a pass over it and a
 * scan per tensor), and a decode of records in device memory from the header
 * words (likewise).  ibp_compress,
 * ibp_decompress and ibp_gather_decompress of such tensors, and
 * ibp_packed_offsets, return IBP_ERR_UNSUPPORTED while `stream` is capturing
 * a HIP graph; single-tile calls may be captured.
 */
#ifndef IBP_H
#define IBP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ibp_status {
    IBP_OK = 0,
    IBP_ERR_INVALID_ARG = -1, /* bad size, pointer kind or parameter */
    IBP_ERR_UNSUPPORTED = -2, /* valid format this GPU path does not implement */
    IBP_ERR_DEVICE = -3,      /* a HIP call failed */
    IBP_ERR_NOMEM = -4,       /* device or host allocation failed */
    IBP_ERR_CORRUPT = -5,     /* a compressed slot holds no valid record */
    IBP_ERR_RANGE = -6,       /* a gather id lies outside [0, n_slots) */
    IBP_ERR_TOO_LARGE = -7    /* more tiles than ibp_decompress_noalloc's static scratch holds */
} ibp_status;

typedef struct ibp_meta_s* ibp_meta_t; /* opaque, owned by the library */

typedef struct ibp_params {
    uint64_t tensor_bytes; /* L: multiple of 4; multiple of W/8 and of M/8        */
    uint32_t chunk_bits;   /* W: 32, 64, 128, 256, 512 or 1024                    */
    uint32_t period_bits;  /* M: multiple of W that divides 8L, at most 2^20      */
    double threshold;      /* T in (0.5, 1]; read by ibp_build_metadata only      */
} ibp_params;

/* Derived facts about a handle's metadata. */
typedef struct ibp_meta_info {
    uint64_t invariant_bits;    /* popcount(Mask) over the M-bit period            */
    uint64_t min_record_bytes;  /* record bytes when every chunk matches           */
    uint32_t max_runs;          /* most runs of kept (unmasked) bits in one word   */
    uint32_t uniform;           /* 1 when every 32-bit Mask/Bitval word is equal   */
} ibp_meta_info;

/* Step 1, preprocessing (FR/KO summary, "Algorithme central" step 1).
 * sample: n_sample tensors of L bytes, contiguous, device or pinned.  Every
 * M-bit block of the sample is one observation; bit position j (0 <= j < M)
 * is invariant when at least K = ceil(T * n_obs) observations agree on it
 * (product rounded to nearest in IEEE double, then ceiling), and Bitval
 * keeps the agreed value there (0 elsewhere).  The histogram runs on the GPU;
 * the call then waits for `stream` and keeps a host copy of Mask/Bitval, so
 * it is synchronous.  n_sample * 8L / M must lie in [1, 2^32).  *out
 * receives a new handle bound to the current HIP device. */
ibp_status ibp_build_metadata(const ibp_params* params, const void* sample, uint64_t n_sample,
                              ibp_meta_t* out, hipStream_t stream);

/* A handle from Mask/Bitval given in host memory (M/32 words each; Bitval
 * bits outside Mask must be 0).  Lets metadata be saved and reused for a
 * whole dataset (FR/KO summary, step 1, last bullet).  Synchronous. */
ibp_status ibp_meta_create(const ibp_params* params, const uint32_t* mask, const uint32_t* bitval,
                           ibp_meta_t* out, hipStream_t stream);

/* Copies the parameters and Mask/Bitval (M/32 words each) to host memory;
 * any output pointer may be NULL. */
ibp_status ibp_meta_get(ibp_meta_t meta, ibp_params* params, uint32_t* mask, uint32_t* bitval);

ibp_status ibp_meta_get_info(ibp_meta_t meta, ibp_meta_info* info);

/* Tuning: bytes of a compressed slot that decode reads before it has seen
 * the record header (a record's length is known only from its header, so a
 * second read fetches the rest).  0 restores the default: the largest
 * 256-byte-aligned prefix no record can be shorter than, but at least 256
 * bytes -- or fewer whole 128-byte lines when the median record of the
 * metadata sample fits in them -- or the whole slot when the shortest
 * possible record spans all but at most 1/16 of the slot's 128-byte lines.
 * Rounded up to a multiple of 16 bytes and to at least the header; capped at
 * the slot.  Affects later decode calls on any stream, except decodes of
 * tensors of at most 1 KiB from slots in GPU memory in launches of at most
 * 128 rows per compute unit, which read each slot whole in one pass. */
ibp_status ibp_meta_set_first_read(ibp_meta_t meta, uint64_t bytes);

/* Waits for all work on the handle's GPU, then frees the handle. */
ibp_status ibp_meta_destroy(ibp_meta_t meta);

/* Step 2, compression (FR/KO summary, "Algorithme central" step 2, and
 * "Intégration au système": fixed slots and a bitmask in GPU memory).
 * src: n_tensors tensors of L bytes (device or pinned).  dst_slots:
 * n_tensors slots of L bytes (device or pinned), must not overlap src.
 * bitmask: device, ceil(n_tensors/32) words; bits 0..n_tensors-1 are
 * written, later bits of the last word are left as they were.
 * stored_bytes: device or NULL; entry t = 4*ceil(R/32) for a compressed
 * slot, L for a raw one. */
ibp_status ibp_compress(ibp_meta_t meta, const void* src, uint64_t n_tensors, void* dst_slots,
                        uint32_t* bitmask, uint64_t* stored_bytes, hipStream_t stream);

/* Step 3, decompression (FR/KO summary, "Algorithme central" step 3):
 * tensor t of dst (device, n_tensors * L bytes) <- slot t of slots (device
 * or pinned).  Only the record prefix of a compressed slot is read.  A
 * compressed slot whose header has non-zero padding bits or implies
 * 4*ceil(R/32) >= L latches IBP_ERR_CORRUPT; its output bytes are then
 * unspecified. */
ibp_status ibp_decompress(ibp_meta_t meta, const void* slots, const uint32_t* bitmask,
                          uint64_t n_tensors, void* dst, hipStream_t stream);

/* Gather on decode: row i of dst (device, n_ids * L bytes) <- slot ids[i]
 * of slots (n_slots slots, device or pinned).  ids: device int64, repeats
 * allowed.  An id outside [0, n_slots) latches IBP_ERR_RANGE and leaves that
 * row unspecified; corrupt records as for ibp_decompress. */
ibp_status ibp_gather_decompress(ibp_meta_t meta, const void* slots, uint64_t n_slots,
                                 const uint32_t* bitmask, const int64_t* ids, uint64_t n_ids,
                                 void* dst, hipStream_t stream);

/* ibp_decompress for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, contract and output as ibp_decompress.  It calls no
 * hipMalloc/hipFree: the start-bit scratch of tensors longer than one tile
 * (L > 8 KiB) lives in one static device array of IBP_NOALLOC_SCRATCH_BYTES
 * per GPU, part of the library's code object and held until the process
 * ends (its address is looked up with hipGetSymbolAddress on the first call
 * on each device).  Each call zeroes the part it uses with fill kernels on
 * `stream` (no memset), so a call may be captured and replayed.  At most
 * IBP_NOALLOC_MAX_TILES tiles per call, a tile being 8 KiB of one tensor
 * (n_tensors * ceil(L / 8192) when L > 8192); beyond that the call returns
 * IBP_ERR_TOO_LARGE before anything is queued.  Every call on a GPU shares
 * its array: calls that overlap in time on one GPU (other streams, other
 * handles, other host threads) race on it and their outputs are then
 * unspecified; calls queued on one stream run one after the other. */
#define IBP_NOALLOC_SCRATCH_BYTES (1u << 20)
#define IBP_NOALLOC_MAX_TILES (IBP_NOALLOC_SCRATCH_BYTES / 8u - 32u)
ibp_status ibp_decompress_noalloc(ibp_meta_t meta, const void* slots, const uint32_t* bitmask,
                                  uint64_t n_tensors, void* dst, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Packed cache (FR/KO summary, "Intégration au système": in the GPU software
 * cache of GNN frameworks, compressing the cached tensors raises how many of
 * them fit).  Instead of fixed L-byte slots, the items -- what slot t would
 * hold: the record when 4*ceil(R/32) < L, else the raw tensor -- are stored
 * back to back.  Item t spans bytes [offsets[t], offsets[t+1]) of the buffer;
 * offsets[0] = 0 and offsets[t+1] = offsets[t] + the item's bytes rounded up
 * to a multiple of 16 (the bytes after an item up to the next offset are
 * zero).  offsets: device memory, n + 1 uint64 entries, 8-byte aligned.  The
 * bitmask is the same as for slots.
 *
 * These calls need L to be a multiple of 16 and at most 8 KiB, 16-byte
 * aligned data pointers, and per-position tables that fit the kernels' LDS
 * (every workload shape of the benchmark does); otherwise they return
 * IBP_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */

/* offsets <- the item offsets of the n_tensors tensors at src (device or
 * pinned); offsets[n_tensors] is the buffer size ibp_compress_packed needs.
 * Reads src once (the record lengths only).  Asynchronous. */
ibp_status ibp_packed_offsets(ibp_meta_t meta, const void* src, uint64_t n_tensors, uint64_t* offsets,
                              hipStream_t stream);

/* Writes item t of src at dst + offsets[t] (dst: device or pinned, capacity
 * bytes, must not overlap src) and bitmask bits 0..n_tensors-1.  offsets
 * must come from ibp_packed_offsets for the same src and handle: an item
 * whose offsets disagree with its length is not written and latches
 * IBP_ERR_CORRUPT, one that would end past capacity latches IBP_ERR_RANGE. */
ibp_status ibp_compress_packed(ibp_meta_t meta, const void* src, uint64_t n_tensors, const uint64_t* offsets,
                               void* dst, uint64_t capacity, uint32_t* bitmask, hipStream_t stream);

/* Tensor t of dst (device, n_items * L bytes) <- item t of the packed
 * buffer buf (device or pinned, buf_bytes bytes).  Each item is read whole
 * in one pass, its length being known from the offsets.  An item whose
 * offsets are not 16-byte multiples, pass buf_bytes, exceed L rounded up to
 * 16, or do not hold its record (or, raw, the whole tensor) latches
 * IBP_ERR_CORRUPT; no byte outside [offsets[t], offsets[t+1]) is read. */
ibp_status ibp_decompress_packed(ibp_meta_t meta, const void* buf, uint64_t buf_bytes, const uint64_t* offsets,
                                 const uint32_t* bitmask, uint64_t n_items, void* dst, hipStream_t stream);

/* Gather on decode from a packed buffer: row i of dst <- item ids[i]
 * (device int64, repeats allowed; an id outside [0, n_items) latches
 * IBP_ERR_RANGE). */
ibp_status ibp_gather_decompress_packed(ibp_meta_t meta, const void* buf, uint64_t buf_bytes,
                                        const uint64_t* offsets, uint64_t n_items, const uint32_t* bitmask,
                                        const int64_t* ids, uint64_t n_ids, void* dst, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Headers in GPU memory ("Intégration au système" keeps the bitmask of
 * compressed slots in GPU memory; this layout keeps each compressed tensor's
 * header words there too).  Zero-copy reads of pinned host memory move whole
 * 128-byte lines, so a record of 4 + 128*j bytes costs j + 1 lines while its
 * payload alone costs j; with the header in GPU memory the decoder also knows
 * the payload length before it reads the slot, and reads it in one pass.
 *
 * Same compressed/raw decision as ibp_compress.  headers: device memory,
 * n * hw uint32 (hw = ceil(n_chunks/32), at most 4, i.e. at most 128 chunks
 * per tensor), 4-byte aligned; entry t*hw .. t*hw+hw-1 holds tensor t's
 * header words, zero for a raw tensor.  Slot t holds the record's payload
 * words (the record minus its header) when compressed, else the tensor; slot
 * bytes after the payload are unspecified.  stored_bytes (device or NULL):
 * payload bytes, or L when raw.  Needs L a multiple of 16 and at most 8 KiB,
 * 16-byte aligned data pointers and tables that fit the kernels' LDS;
 * otherwise IBP_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------- */
ibp_status ibp_compress_split(ibp_meta_t meta, const void* src, uint64_t n_tensors, void* dst_slots,
                              uint32_t* headers, uint32_t* bitmask, uint64_t* stored_bytes, hipStream_t stream);

/* Tensor t of dst (device) <- slot t (device or pinned) with its header
 * words from headers.  A compressed tensor whose header padding bits are set
 * or whose header implies 4*ceil(R/32) >= L latches IBP_ERR_CORRUPT. */
ibp_status ibp_decompress_split(ibp_meta_t meta, const void* slots, const uint32_t* headers,
                                const uint32_t* bitmask, uint64_t n_tensors, void* dst, hipStream_t stream);

/* Gather on decode in that layout: row i of dst <- tensor ids[i] (device
 * int64; an id outside [0, n_slots) latches IBP_ERR_RANGE). */
ibp_status ibp_gather_decompress_split(ibp_meta_t meta, const void* slots, uint64_t n_slots,
                                       const uint32_t* headers, const uint32_t* bitmask, const int64_t* ids,
                                       uint64_t n_ids, void* dst, hipStream_t stream);

/* Waits for `stream`, returns the first error latched by a kernel of this
 * handle since the last ibp_check (IBP_OK if none) and clears it:
 * IBP_ERR_RANGE, IBP_ERR_CORRUPT, or IBP_ERR_DEVICE when a tile gave up
 * waiting for its predecessor in the look-back (its tensor's output is then
 * unspecified). */
ibp_status ibp_check(ibp_meta_t meta, hipStream_t stream);

const char* ibp_status_string(ibp_status status);

#ifdef __cplusplus
}
#endif
#endif
