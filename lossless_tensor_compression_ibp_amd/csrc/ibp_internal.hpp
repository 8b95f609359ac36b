// ibp_internal.hpp -- structures shared by the host side of libibp and its
// gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ibp {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kWavesPerBlock = 4;   // independent waves per workgroup
constexpr int kMaxRuns = 16;        // a 32-bit word has at most 16 runs of ones
constexpr int kPlanes = 11;         // bit planes of a per-chunk k (k <= 1024)
constexpr uint32_t kMaxTileWords = 2048;  // largest tile one wave owns
constexpr uint64_t kMaxLdsTableBytes = 48 * 1024;  // per-position tables staged in LDS
constexpr uint64_t kMaxLdsPlaneBytes = 16 * 1024;  // header bit planes staged in LDS
constexpr uint64_t kMaxLdsPerBlock = 64 * 1024;    // dynamic LDS of one workgroup
constexpr uint64_t kLdsPerCu = 160 * 1024;         // gfx950 LDS per compute unit

// Derived per-position tables in device memory (structure of arrays; every
// array has Mw entries unless stated).  Position i of the metadata period is
// 32-bit word i of Mask/Bitval.
struct Tables {
    const uint32_t* m;       // Mask word
    const uint32_t* b;       // Bitval word
    const uint32_t* kd;      // k | d0 << 8 | d1 << 16 | d2 << 24
    const uint32_t* dx;      // [4][Mw]: run shifts d3.. packed 4 per word
    const uint32_t* r;       // [kMaxRuns][Mw]: run masks, output positions
    const uint32_t* planes;  // [Ne][kPlanes]: bit planes of per-chunk k
};

// Shape of one launch: the tensor geometry plus how it is cut into tiles.
struct Geo {
    uint64_t L;              // tensor (and slot) bytes
    uint64_t n_words;        // L / 4
    uint64_t n_chunks;       // 8L / W
    uint64_t hdr_words;      // ceil(n_chunks / 32)
    uint32_t Mw;             // period in words (M / 32)
    uint32_t Pc;             // period in chunks (M / W)
    uint32_t log2g;          // log2(W / 32)
    uint32_t G;              // gcd(32, Pc)
    uint32_t np;             // bit planes worth scanning (<= kPlanes)
    uint32_t k1;             // Pc == 1: the k every chunk removes
    uint32_t tile_words;     // words per tile (multiple of 64 * 32 >> ... see host)
    uint64_t tiles_per_tensor;
    uint32_t spec_words;     // first-read words of a single-tile record (multiple of 4)
    uint32_t aligned16;      // slot base and L allow 16-byte vector access
    uint32_t src_in_hbm;     // what the launch reads (stored items, or the encode's source) is in device memory
    uint32_t dst_in_hbm;     // the encode's slots are in device memory
};

// Decoupled look-back state for multi-tile tensors.  A status word packs
// flag (2 bits) | epoch (20 bits) | value (42 bits).  The ticket counter is
// set to zero by a fill kernel on the launch's stream right before each
// launch, so the tiles of a launch take tickets 0, 1, 2, ... in stream order
// and no counter state lives on the host.
struct LookBack {
    unsigned long long* status;  // one per tile of the launch
    uint32_t* ticket;            // dynamic tile counter (zero at launch)
    uint32_t epoch;              // 1 .. 2^20-1, distinct from stale entries
    uint64_t* totals;            // per output tensor: record bits (encode)
    uint32_t* err;               // error latch of the handle
};

// A look-back wait gives up after this many polls of one predecessor's
// status word (each poll is an atomic load and a short sleep, so several
// seconds; a predecessor holds an earlier ticket and is resident or done, so
// a legitimate wait lasts microseconds).  The tile then latches kErrStall and
// publishes kLookbackPoison as its inclusive value, which every later tile
// of the tensor rejects before it touches memory.
constexpr uint32_t kLookbackPolls = 1u << 22;
constexpr uint64_t kLookbackPoison = 1ull << 41;

// The decode of a tensor longer than one tile gives each wave a group of up
// to this many consecutive tiles of one tensor (one status word per group).
// Records read over the host link: the look-back chains groups, and a
// workgroup takes one ticket for its waves' groups; measured on MI355X (32
// llm_bf16 layers of 90 MB, 8 KiB tiles) 2 / 4 / 8 / 16 tiles per group
// decode a layer zero-copy from pinned memory in 1,277 / 1,268 / 1,255 /
// 1,270 us, and 8 is kept (1,263 / 1,251 us at 4 / 8 with the current
// kernel).  Records in HBM take their start bits from a header pass instead;
// there 2 / 3 / 4 / 8 / 16 tiles per group decode all 32 layers in
// 918 / 950 / 899-909 / 955-961 / 1,046 us: groups of 4 keep 16 waves per CU
// resident (LDS: a 1 KiB header area and an 8 KiB payload buffer per wave)
// against 12 with groups of 8.
#ifndef IBP_DECODE_TILES_PER_GROUP
#define IBP_DECODE_TILES_PER_GROUP 8
#endif
#ifndef IBP_DECODE_TILES_PER_GROUP_HBM
#define IBP_DECODE_TILES_PER_GROUP_HBM 4
#endif
constexpr uint32_t kDecodeTilesPerGroup = IBP_DECODE_TILES_PER_GROUP;
constexpr uint32_t kDecodeTilesPerGroupHbm = IBP_DECODE_TILES_PER_GROUP_HBM;
// Waves per workgroup of the group decode.
#ifndef IBP_DECODE_GROUP_WAVES
#define IBP_DECODE_GROUP_WAVES 4
#endif
constexpr int kGroupWaves = IBP_DECODE_GROUP_WAVES;
__host__ __device__ constexpr uint64_t tile_groups(uint64_t tiles_per_tensor, uint32_t tiles_per_group) {
    return (tiles_per_tensor + tiles_per_group - 1) / tiles_per_group;
}
// Tiles per group of a decode whose stored records are (not) in device memory.
__host__ __device__ constexpr uint32_t decode_group_tiles(bool src_in_hbm) {
    return src_in_hbm ? kDecodeTilesPerGroupHbm : kDecodeTilesPerGroup;
}
// Words per tile of a tensor longer than kMaxTileWords, for a decode whose
// records are read over the host link, and for one whose records are in
// device memory.  The record format does not depend on the tile size.  From
// HBM, 1,024-word tiles (fewer prefetch registers, half the LDS per wave)
// decoded the 32 llm_bf16 layers in 937-940 us in groups of 4 or 8 and
// 1,002 us in groups of 16, against 895 us with 2,048-word tiles in groups
// of 4 (916 us in groups of 2).
#ifndef IBP_DECODE_TILE_WORDS_HBM
#define IBP_DECODE_TILE_WORDS_HBM 2048
#endif
constexpr uint32_t kLongTileWordsDecode = 2048;
constexpr uint32_t kLongTileWordsDecodeHbm = IBP_DECODE_TILE_WORDS_HBM;
static_assert(kLongTileWordsDecodeHbm % 256 == 0 && kLongTileWordsDecodeHbm <= kMaxTileWords, "tile words");
__host__ __device__ constexpr uint32_t decode_tile_words(bool src_in_hbm) {
    return src_in_hbm ? kLongTileWordsDecodeHbm : kLongTileWordsDecode;
}
// Bitmask words one workgroup of the small-tensor encode can cover: it takes
// at most 16 waves x kMaxItemsPerWave tensors (the launch plan guarantees it),
// which span at most 5 words.
constexpr uint32_t kEncBlockBitWords = 8;

// Words per tile of a tensor longer than kMaxTileWords, for the encode (over
// the host link it measured faster than 2,048-word tiles).
constexpr uint32_t kLongTileWordsEncode = 1024;
// Tiles per group of an encode whose source is in device memory: a first pass
// sums each group's payload bits, a per-tensor scan turns the sums into start
// bits, and one wave then encodes the group's tiles in order.
#ifndef IBP_ENCODE_TILES_PER_GROUP_HBM
#define IBP_ENCODE_TILES_PER_GROUP_HBM 4
#endif
constexpr uint32_t kEncodeTilesPerGroupHbm = IBP_ENCODE_TILES_PER_GROUP_HBM;

// Whether an encode of tensors longer than one tile takes the two-pass path
// (source in device memory, 16-byte aligned) rather than look-back per tile;
// it needs one status word per group instead of one per tile.
inline bool encode_two_pass(const Geo& g) { return g.src_in_hbm && g.aligned16; }
inline uint64_t encode_status_words(const Geo& g, uint64_t n_tensors) {
    return n_tensors * (encode_two_pass(g) ? tile_groups(g.tiles_per_tensor, kEncodeTilesPerGroupHbm)
                                           : g.tiles_per_tensor);
}

// Exclusive start bits, `base` first, of the n_tensors * gpt group bit counts
// in `bits` (in place; gpt consecutive groups per tensor).
hipError_t launch_group_scan(uint64_t n_tensors, uint64_t gpt, uint64_t base, uint64_t* bits, hipStream_t s);

enum DeviceError : uint32_t { kErrNone = 0, kErrCorrupt = 5, kErrRange = 6, kErrStall = 7 };

// Where tensor t's stored item lives.  offsets == nullptr: fixed slots, slot
// t at byte t * L.  Otherwise the packed cache layout: item t spans bytes
// [offsets[t], offsets[t+1]) of a buffer of `bytes` bytes, each item starting
// on a 16-byte boundary and its length a multiple of 16.
struct Items {
    const uint64_t* offsets;
    uint64_t bytes;
};

// Summary written by the table builder, read back by the host.
struct Summary {
    uint32_t max_runs;
    uint32_t max_chunk_k;
    uint32_t uniform;
    uint32_t pad;
    unsigned long long invariant_bits;
    unsigned long long removed_per_period;  // sum of k over the period
};

// Launch shape of a persistent kernel: waves per workgroup, workgroups, and
// dynamic LDS per workgroup.
struct PersistentPlan {
    uint32_t wpb = 0;
    uint32_t blocks = 0;
    size_t shm = 0;
};

// Chooses the waves per workgroup (4, 8, 12 or 16, within the kernel's launch
// bounds) that keeps the most waves resident per compute unit, given LDS
// shared by a workgroup (head_bytes), LDS per wave (wave_bytes), the kernel's
// VGPR count, the LDS limits of the device and at most max_waves_per_simd
// resident waves per SIMD.
// blocks = min(items / wpb, max(workgroups that fill the device,
// items / (wpb * max_items))).  Returns false when no shape fits.
//
// max_items: a wave of a persistent launch takes at most this many items;
// longer launches get more workgroups than fit at once.  Measured on MI355X
// with the 262,144 4 KiB KV pages in HBM (64 pages per resident wave
// otherwise): the encode moves 2.20 / 2.36 / 2.53-2.56 / 2.57 / 2.52 TB/s of
// input at 2 / 4 / 8 / 16 / 32 pages per wave (kMaxItemsPerWave, 8); the
// decode takes 474 / 369 / 359-361 / 354-357 / 360 / 363 / 361 us at
// 1 / 2 / 3 / 4 / 5 / 6 / 8 pages per wave (kDecodeItemsPerWave, 4), where
// every workgroup stages 21 KiB of tables for its waves' pages.  512-byte
// and 1 KiB rows in HBM (dense_gnn, the packed cache) and zero-copy gathers
// of 65,536 rows of 512 bytes decode alike at 4 to 8.  A plain copy of 4 KiB pages shows
// the same trade: persistent waves striding over the pages move
// 5.7-5.9 TB/s, one wave per page 6.3 TB/s.
#ifndef IBP_MAX_ITEMS_PER_WAVE
#define IBP_MAX_ITEMS_PER_WAVE 8
#endif
constexpr uint64_t kMaxItemsPerWave = IBP_MAX_ITEMS_PER_WAVE;
static_assert(16 * kMaxItemsPerWave + 31 <= 32ull * kEncBlockBitWords,
              "a workgroup's tensors must fit the encode's LDS bitmask words");
#ifndef IBP_DECODE_ITEMS_PER_WAVE
#define IBP_DECODE_ITEMS_PER_WAVE 4
#endif
constexpr uint64_t kDecodeItemsPerWave = IBP_DECODE_ITEMS_PER_WAVE;
bool plan_persistent(const void* kernel, size_t head_bytes, size_t wave_bytes, uint32_t cu_count,
                     uint64_t n_items, PersistentPlan* plan, uint32_t max_waves_per_simd = 8,
                     uint64_t max_items = kMaxItemsPerWave);

// Kernel launchers.  All return hipError_t of the launch.
hipError_t launch_fill_u32(uint32_t* p, uint64_t n, uint32_t v, hipStream_t s);
hipError_t launch_meta_hist(const uint32_t* sample, uint64_t n_words, uint32_t Mw, uint32_t* counts,
                            hipStream_t s);
hipError_t launch_meta_finalize(const uint32_t* counts, uint32_t Mw, uint64_t n_obs, uint64_t K,
                                uint32_t* mask, uint32_t* bitval, hipStream_t s);
hipError_t launch_tables(const uint32_t* mask, const uint32_t* bitval, uint32_t Mw, uint32_t Pc,
                         uint32_t g, uint32_t G, uint32_t* kd, uint32_t* dx, uint32_t* r,
                         uint32_t* planes, Summary* summary, hipStream_t s);
hipError_t launch_encode(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta, const void* src,
                         uint64_t n_tensors, void* slots, uint32_t* bitmask, uint64_t* stored, const LookBack* lb,
                         uint32_t cu_count, hipStream_t s);
hipError_t launch_decode(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta, const void* slots,
                         uint64_t n_slots, const uint32_t* bitmask, const int64_t* ids, uint64_t n_out,
                         void* dst, uint32_t* err, const LookBack* lb, uint32_t cu_count, hipStream_t s,
                         const Items* items = nullptr, const uint32_t* headers = nullptr);

// Packed cache.  These run only on the persistent small-tensor kernels
// (16-byte aligned tensors of at most kMaxTileWords words whose tables fit in
// LDS); packed_supported() says whether a geometry qualifies.
bool packed_supported(const Geo& geo, uint32_t runs, bool uniform_meta);         // encode side
bool packed_decode_supported(const Geo& geo, uint32_t runs, bool uniform_meta);  // decode side
// sizes[t] <- bytes of tensor t's item rounded up to 16 (record or raw).
hipError_t launch_item_sizes(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta, const void* src,
                             uint64_t n_tensors, uint64_t* sizes, uint32_t cu_count, hipStream_t s);
// Items of src written at their offsets (packed), bitmask as for slots;
// items whose offsets disagree with their length or pass the buffer's end
// are skipped and latch an error.
hipError_t launch_encode_packed(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta,
                                const void* src, uint64_t n_tensors, void* dst, const Items& items,
                                uint32_t* bitmask, uint32_t* err, uint32_t cu_count, hipStream_t s);
// Headers in GPU memory: header words of each compressed tensor in an array
// beside the bitmask, the payload alone in the slot.  At most
// kMaxSplitHeaderWords header words (128 chunks) per tensor, persistent
// small-tensor kernels only.
constexpr uint64_t kMaxSplitHeaderWords = 4;
bool split_supported(const Geo& geo, uint32_t runs, bool uniform_meta);
hipError_t launch_encode_split(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta, const void* src,
                               uint64_t n_tensors, void* slots, uint32_t* headers, uint32_t* bitmask,
                               uint64_t* stored, uint32_t cu_count, hipStream_t s);
// offsets[1..n] hold sizes on entry and their inclusive prefix sums on exit;
// offsets[0] <- 0.  One look-back entry per block of kScanBlock sizes.
constexpr uint32_t kScanPerLane = 8;
constexpr uint32_t kScanBlock = kScanPerLane * kWave;
hipError_t launch_scan_sizes(uint64_t* offsets, uint64_t n, const LookBack& lb, hipStream_t s);
uint64_t scan_waves(uint64_t n);

}  // namespace ibp
