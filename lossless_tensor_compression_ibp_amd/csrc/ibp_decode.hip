// ibp_decode.hip -- step 3 of Invariant Bit Packing on gfx950: decompression.
//
// Method: FR summary ("Résumé Technique : Réduire le goulot d'étranglement de
// la mémoire GPU par la compression sans perte pour le ML") and KO summary
// ("Reducing the GPU Memory Bottleneck with Lossless Compression for ML --
// Extended"), section "Algorithme central" / "핵심 알고리즘", step 3: the
// lanes of a wave load a contiguous compressed segment together into a
// shared workspace, scan the chunk sizes for each chunk's start bit, and
// rebuild their chunks by putting Bitval's invariant bits back; loads are
// issued ahead of the decode to hide link latency.  Section "Intégration au
// système": a bitmask in GPU memory says which fixed-size slots hold a record,
// and only the record prefix of a slot is read.
//
// Layout of the work: one wave64 decodes one tile (all of a tensor of at most
// 2048 words, or a 2048-word tile of a longer one).  A lane rebuilds four
// consecutive 32-bit words per step (256 words per wave step), so a step
// costs one DPP scan and one dwordx4 store per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "ibp_device.hpp"
#include "ibp_internal.hpp"

namespace ibp {

// Step shapes of decode_tile.
constexpr int kTileOneStep = 0, kTileMultiStep = 1, kTileHalfStep = 2;

// One step of decode_tile: lane words lw0 .. lw0+3 (256 words per wave).
// FULL: every lane's four words lie inside the tile, so the step needs no
// bounds checks (every step but a ragged last one).
template <int RUNS, bool MW4, bool FULL, class Tab>
__device__ __forceinline__ void decode_step(const Tab& tab, const Geo& geo, const uint32_t* hdr,
                                            const uint32_t* pay, uint32_t lw0, uint32_t pos0, uint32_t nw,
                                            uint32_t* carry, uint32_t* __restrict__ out, bool vec,
                                            bool full_rt = false) {
    constexpr bool UNI = IsUniformTab<Tab>::value;
    const uint32_t Mw = geo.Mw;
    const uint32_t lg = geo.log2g;
    uint32_t pos[4], kd[4], bv[4];
    uint32_t rr[RUNS > 0 ? RUNS : 1][4];
    if constexpr (UNI) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pos[j] = 0;
            kd[j] = tab.kdw(0);
            bv[j] = tab.bw(0);
        }
    } else if constexpr (MW4) {
        const u32x4 k4 = tab.kdw4(pos0), b4 = tab.bw4(pos0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pos[j] = pos0 + j;
            kd[j] = k4[j];
            bv[j] = b4[j];
        }
    } else {
        pos[0] = pos0;
#pragma unroll
        for (int j = 1; j < 4; ++j) pos[j] = (pos[j - 1] + 1 == Mw) ? 0u : pos[j - 1] + 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            kd[j] = tab.kdw(pos[j]);
            bv[j] = tab.bw(pos[j]);
        }
    }
    const uint32_t c0 = lw0 >> lg;
    const uint32_t hsh = hdr[c0 >> 5] >> (c0 & 31u);
    uint32_t p[4], size[4];
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        p[j] = (hsh >> ((uint32_t)j >> lg)) & 1u;
        const uint32_t sz = p[j] ? 32u - (kd[j] & 63u) : 32u;
        size[j] = (FULL || full_rt || lw0 + j < nw) ? sz : 0u;
        tot += size[j];
    }
    const uint32_t incl = wave_incl_scan(tot);
    uint32_t off = *carry + incl - tot;
    *carry += lane_value(incl, kWave - 1);
    // run masks (and shifts of runs past the third) of the lane's four positions
    if constexpr (MW4 && !UNI) {
#pragma unroll
        for (int r = 0; r < RUNS; ++r) {
            const u32x4 v = tab.rw4(r, pos0);
#pragma unroll
            for (int j = 0; j < 4; ++j) rr[r][j] = v[j];
        }
    } else {
#pragma unroll
        for (int r = 0; r < RUNS; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) rr[r][j] = tab.rw(r, pos[j]);
    }
    uint32_t x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t q = off >> 5;
        const uint32_t f = funnel(pay[q + 1], pay[q], off);
        uint32_t dep = bv[j];
#pragma unroll
        for (int r = 0; r < RUNS; ++r) dep |= (f << (tab.dw(r, pos[j], kd[j]) & 31u)) & rr[r][j];
        x[j] = p[j] ? dep : f;
        off += size[j];
    }
    if (vec && (FULL || full_rt || lw0 + 3 < nw)) {
        __builtin_nontemporal_store(u32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<u32x4*>(out + lw0));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (FULL || lw0 + j < nw) out[lw0 + j] = x[j];
    }
}

// The same step for tensors of at most 128 words: lane words lw0, lw0 + 1
// (128 words per wave), so no lane idles on a 512-byte row as it would with
// four words per lane.  MW4: Mw is a multiple of 4, so a lane's two positions
// are consecutive and read as one 8-byte vector.
template <int RUNS, bool MW4, class Tab>
__device__ __forceinline__ void decode_step2(const Tab& tab, const Geo& geo, const uint32_t* hdr,
                                             const uint32_t* pay, uint32_t lw0, uint32_t pos0, uint32_t nw,
                                             uint32_t* carry, uint32_t* __restrict__ out, bool vec) {
    constexpr bool UNI = IsUniformTab<Tab>::value;
    const uint32_t Mw = geo.Mw;
    const uint32_t lg = geo.log2g;
    uint32_t pos[2], kd[2], bv[2];
    uint32_t rr[RUNS > 0 ? RUNS : 1][2];
    if constexpr (UNI) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            pos[j] = 0;
            kd[j] = tab.kdw(0);
            bv[j] = tab.bw(0);
        }
    } else if constexpr (MW4) {
        const u32x2 k2 = tab.kdw2(pos0), b2 = tab.bw2(pos0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            pos[j] = pos0 + j;
            kd[j] = k2[j];
            bv[j] = b2[j];
        }
    } else {
        pos[0] = pos0;
        pos[1] = (pos0 + 1 == Mw) ? 0u : pos0 + 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            kd[j] = tab.kdw(pos[j]);
            bv[j] = tab.bw(pos[j]);
        }
    }
    const uint32_t c0 = lw0 >> lg;
    const uint32_t hsh = hdr[c0 >> 5] >> (c0 & 31u);
    uint32_t p[2], size[2];
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        p[j] = (hsh >> ((uint32_t)j >> lg)) & 1u;
        size[j] = lw0 + j < nw ? (p[j] ? 32u - (kd[j] & 63u) : 32u) : 0u;
        tot += size[j];
    }
    const uint32_t incl = wave_incl_scan(tot);
    uint32_t off = *carry + incl - tot;
    *carry += lane_value(incl, kWave - 1);
    if constexpr (MW4 && !UNI) {
#pragma unroll
        for (int r = 0; r < RUNS; ++r) {
            const u32x2 v = tab.rw2(r, pos0);
            rr[r][0] = v[0];
            rr[r][1] = v[1];
        }
    } else {
#pragma unroll
        for (int r = 0; r < RUNS; ++r)
#pragma unroll
            for (int j = 0; j < 2; ++j) rr[r][j] = tab.rw(r, pos[j]);
    }
    uint32_t x[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t q = off >> 5;
        const uint32_t f = funnel(pay[q + 1], pay[q], off);
        uint32_t dep = bv[j];
#pragma unroll
        for (int r = 0; r < RUNS; ++r) dep |= (f << (tab.dw(r, pos[j], kd[j]) & 31u)) & rr[r][j];
        x[j] = p[j] ? dep : f;
        off += size[j];
    }
    if (vec && lw0 + 1 < nw) {
        __builtin_nontemporal_store(u32x2{x[0], x[1]}, reinterpret_cast<u32x2*>(out + lw0));
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (lw0 + j < nw) out[lw0 + j] = x[j];
    }
}

// Rebuild words [w0, w0 + nw) of a tensor into out.  hdr: participation bits
// of the tile (bit 0 = the tile's first chunk); pay: LDS words holding the
// tile's kept bits, the first at bit `bit0` of pay[0].  Lanes past the end
// contribute size 0.  With `vec`, out + w0 is 16-byte aligned.  MW4: the
// period Mw is a multiple of 4 (and w0 too), so a lane's four positions are
// consecutive and their table entries are read as one 16-byte vector.
// MODE kTileMultiStep: tiles of several 256-word steps get a step body
// compiled without bounds checks (measured 2 % faster on 4 KiB pages);
// kTileOneStep: tiles of at most a few steps keep a single body, whose lower
// register count keeps more waves resident (measured 2.5 % faster on 512-byte
// and 1 KiB rows); kTileHalfStep: tiles of at most 128 words (w0 even) take
// one step of two words per lane.
template <int RUNS, bool MW4, int MODE, class Tab>
__device__ __forceinline__ uint32_t decode_tile(const Tab& tab, const Geo& geo, const uint32_t* hdr,
                                                const uint32_t* pay, uint32_t bit0, uint64_t w0,
                                                uint32_t nw, uint32_t* __restrict__ out, bool vec) {
    constexpr bool UNI = IsUniformTab<Tab>::value;
    const uint32_t lane = lane_id();
    const uint32_t Mw = geo.Mw;
    const uint32_t step_inc = (uint32_t)(4 * kWave) % Mw;
    uint32_t pos0 = UNI ? 0u : (uint32_t)((w0 + 4ull * lane) % Mw);
    uint32_t carry = bit0;
    uint32_t* o = out + w0;
    if constexpr (MODE == kTileHalfStep) {
        decode_step2<RUNS, MW4>(tab, geo, hdr, pay, 2 * lane, UNI ? 0u : (uint32_t)((w0 + 2ull * lane) % Mw), nw,
                                &carry, o, vec);
        return carry;
    } else if constexpr (MODE == kTileOneStep) {
        const uint32_t steps = (nw + 4 * kWave - 1) / (4 * kWave);
        for (uint32_t s = 0; s < steps; ++s) {
            const bool full = (s + 1) * (4 * kWave) <= nw;  // wave-uniform: no lane runs past the end
            decode_step<RUNS, MW4, false>(tab, geo, hdr, pay, s * (4 * kWave) + 4 * lane, pos0, nw, &carry, o, vec,
                                          full);
            if constexpr (!UNI) {
                pos0 += step_inc;
                if (pos0 >= Mw) pos0 -= Mw;
            }
        }
        return carry;
    } else {
        const uint32_t full_steps = nw / (4 * kWave);
        for (uint32_t s = 0; s < full_steps; ++s) {
            decode_step<RUNS, MW4, true>(tab, geo, hdr, pay, s * (4 * kWave) + 4 * lane, pos0, nw, &carry, o, vec);
            if constexpr (!UNI) {
                pos0 += step_inc;
                if (pos0 >= Mw) pos0 -= Mw;
            }
        }
        if (full_steps * (4 * kWave) < nw)
            decode_step<RUNS, MW4, false>(tab, geo, hdr, pay, full_steps * (4 * kWave) + 4 * lane, pos0, nw, &carry,
                                          o, vec);
        return carry;
    }
}

// LDS image of the tables: b, kd, dx rows, r rows (stride Mw), then the
// header bit planes.  Copied once per workgroup.
// A whole tile of TW words (every step full, output 16-byte aligned, w0 a
// multiple of 4): decode_tile with a compile-time step count, so the steps
// unroll into one block with one store each.
template <int RUNS, uint32_t TW, class Tab>
__device__ __forceinline__ void decode_full_tile(const Tab& tab, const Geo& geo, const uint32_t* hdr,
                                                 const uint32_t* pay, uint32_t bit0, uint64_t w0,
                                                 uint32_t* __restrict__ out) {
    constexpr bool UNI = IsUniformTab<Tab>::value;
    const uint32_t lane = lane_id();
    const uint32_t Mw = geo.Mw;
    const uint32_t step_inc = (uint32_t)(4 * kWave) % Mw;
    uint32_t pos0 = UNI ? 0u : (uint32_t)((w0 + 4ull * lane) % Mw);
    uint32_t carry = bit0;
#pragma unroll
    for (uint32_t s = 0; s < TW / (4 * kWave); ++s) {
        decode_step<RUNS, false, true>(tab, geo, hdr, pay, s * (4 * kWave) + 4 * lane, pos0, TW, &carry, out + w0,
                                       true);
        if (!UNI) {
            pos0 += step_inc;
            if (pos0 >= Mw) pos0 -= Mw;
        }
    }
}

template <int RUNS>
__device__ __forceinline__ void stage_tables(const Tables& t, uint32_t Mw, uint32_t n_planes_words,
                                             bool per_position, uint32_t* lds) {
    stage_table_image<dx_rows(RUNS)>(t, 1, per_position ? tab_rows(RUNS) : 0u, Mw, t.planes, n_planes_words, lds);
}

// ---------------------------------------------------------------------------
// Tensors of at most kMaxTileWords words with 16-byte aligned slots and
// output: persistent workgroups, tables staged once in LDS, and per wave a
// software pipeline over its tiles.  All ids and bitmask bits of a wave's
// next 64 tiles are fetched first (one lane per tile); then the first read of
// tile k+1 (the whole slot of a raw tensor, the first spec_words of a record)
// is in flight in registers while tile k is decoded.  STAGE: 16-byte vectors
// per lane of that read; STAGE 0 for tensors of at most 128 words, which one
// vector per lane covers and whose rebuild takes two words per lane.
//
// Packed cache layout (items.offsets set): each lane also fetches its tile's
// item span; every read stays inside that span, and an item whose span does
// not fit its record (or the buffer) latches a corrupt-record error.
//
// SPLIT (headers in GPU memory, at most 4 header words): each lane fetches
// its tile's header words with the bitmask bit and works out the payload
// length from them, so the slot read takes exactly the payload (rounded up
// to 16 bytes) in one pass; the header is put back in LDS beside the payload
// for the rebuild.
// ---------------------------------------------------------------------------
template <int RUNS, bool UNI, bool MW4, int STAGE, bool SPLIT>
__global__ __launch_bounds__(256) void k_decode_small(Tables t, Geo geo, const uint8_t* __restrict__ slots,
                                                      uint64_t n_slots, const uint32_t* __restrict__ bitmask,
                                                      const int64_t* __restrict__ ids, uint64_t n_out,
                                                      uint8_t* __restrict__ dst, uint32_t* err,
                                                      uint32_t buf_words, Items items,
                                                      const uint32_t* __restrict__ headers) {
    extern __shared__ uint32_t smem[];
    const uint32_t lane = lane_id();
    const uint32_t wib = uniform(threadIdx.x / kWave);
    const uint32_t Mw = geo.Mw;
    // LDS: [per-position tables (not for uniform metadata)][bit planes][wave buffers]
    const uint32_t tab_words = UNI ? 0u : tab_rows(RUNS) * Mw;
    const uint32_t planes_words = (geo.Pc / geo.G) * (uint32_t)kPlanes;
    const uint32_t wpb = blockDim.x / kWave;
    const uint64_t stride = (uint64_t)gridDim.x * wpb;
    const uint64_t first = (uint64_t)blockIdx.x * wpb + wib;
    const uint64_t my_tiles = first < n_out ? (n_out - first + stride - 1) / stride : 0;
    // A gather fetches the ids of the wave's first 64 tiles before the tables
    // are staged: the staging loads are issued after it, so waiting for them
    // also covers it, and the two latencies overlap.
    int64_t first_id = -1;
    if (ids && lane < min((uint64_t)kWave, my_tiles)) first_id = ids[first + lane * stride];
    stage_tables<RUNS>(t, Mw, planes_words, !UNI, smem);
    __syncthreads();
    const uint32_t* planes = smem + tab_words;
    uint32_t* buf = smem + ((tab_words + planes_words + 3u) & ~3u) + wib * buf_words;
    const TabArrays ta{smem, smem + Mw, smem + 2 * Mw, smem + (2 + dx_rows(RUNS)) * Mw, Mw};
    TabUniform<RUNS> tu;
    if (UNI) tu = load_uniform<RUNS>(t, Mw);

    const uint32_t nwords = (uint32_t)geo.n_words;
    const uint32_t n4_raw = nwords >> 2;
    const uint32_t n4_spec = geo.spec_words >> 2;
    const uint32_t hw = (uint32_t)geo.hdr_words;
    if (first >= n_out) return;

    // STAGE 0: tensors of at most 128 words (one 16-byte vector per lane is
    // read, and the rebuild takes two words per lane)
    constexpr int kSt = STAGE > 0 ? STAGE : 1;
    constexpr int kTileMode = STAGE >= 4 ? kTileMultiStep : (STAGE == 0 ? kTileHalfStep : kTileOneStep);
    u32x4 st[kSt];
    for (uint64_t base = 0; base < my_tiles; base += kWave) {
        const uint32_t cnt = (uint32_t)min((uint64_t)kWave, my_tiles - base);
        // lane k: id of tile base + k; the first read of tile 0 (the same
        // prefix for raw and compressed slots) goes out before the bitmask
        // bits are fetched, so the two loads overlap
        const bool packed = items.offsets != nullptr;
        int64_t my_tensor = -1;
        bool bad_id = false, bad_item = false;
        uint64_t my_off = 0;
        uint32_t my_len = 0;
        if (lane < cnt) {
            const uint64_t oi = first + (base + lane) * stride;
            const int64_t id = ids ? (base == 0 ? first_id : ids[oi]) : (int64_t)oi;
            if (id >= 0 && (uint64_t)id < n_slots) {
                my_tensor = id;
                if (packed) {
                    const uint64_t a = items.offsets[id], b = items.offsets[id + 1];
                    bad_item = b < a || b > items.bytes || ((a | b) & 15) || b - a > ((geo.L + 15) & ~15ull);
                    if (bad_item) {
                        my_tensor = -1;
                    } else {
                        my_off = a;
                        my_len = (uint32_t)(b - a);
                    }
                }
            } else {
                bad_id = true;
            }
        }
        const uint32_t t_lo = (uint32_t)my_tensor, t_hi = (uint32_t)((uint64_t)my_tensor >> 32);
        const uint32_t o_lo = (uint32_t)my_off, o_hi = (uint32_t)(my_off >> 32);

        auto tensor_of = [&](uint32_t k) __attribute__((always_inline)) -> int64_t {
            return (int64_t)(((uint64_t)lane_value(t_hi, k) << 32) | lane_value(t_lo, k));
        };
        // SPLIT: the bitmask bit and header words of each lane's tile, and
        // from them the payload words its slot read takes
        uint32_t my_comp = 0, my_pw = 0;
        uint32_t h0 = 0, h1 = 0, h2 = 0, h3 = 0;
        bool bad_rec = false;
        if constexpr (SPLIT) {
            if (lane < cnt && my_tensor >= 0) {
                my_comp = (bitmask[(uint64_t)my_tensor >> 5] >> ((uint64_t)my_tensor & 31)) & 1u;
                if (my_comp) {
                    const uint32_t* hp = headers + (uint64_t)my_tensor * hw;
                    uint32_t hv[4] = {0u, 0u, 0u, 0u};
                    uint32_t rem = 0;
#pragma unroll
                    for (uint32_t j = 0; j < 4; ++j) {
                        if (j < hw) {
                            uint32_t h = hp[j];
                            hv[j] = h;
                            if (j == hw - 1) {
                                const uint32_t valid = (uint32_t)(geo.n_chunks - 32ull * j);
                                if (valid < 32) {
                                    if (h >> valid) bad_rec = true;
                                    h &= (1u << valid) - 1u;
                                }
                            }
                            rem += removed_bits_pl(planes, geo, j, h);
                        }
                    }
                    const uint64_t R = 32ull * hw + 32ull * nwords - rem;
                    const uint32_t words = (uint32_t)((R + 31) / 32);
                    if (4ull * words >= geo.L) bad_rec = true;
                    if (bad_rec) {
                        my_tensor = -1;
                    } else {
                        my_pw = words - hw;
                        h0 = hv[0];
                        h1 = hv[1];
                        h2 = hv[2];
                        h3 = hv[3];
                    }
                }
            }
        }
        const uint32_t t_lo2 = (uint32_t)my_tensor, t_hi2 = (uint32_t)((uint64_t)my_tensor >> 32);
        auto tensor_of2 = [&](uint32_t k) __attribute__((always_inline)) -> int64_t {
            if constexpr (!SPLIT) return tensor_of(k);
            return (int64_t)(((uint64_t)lane_value(t_hi2, k) << 32) | lane_value(t_lo2, k));
        };

        // byte offset of tile k's slot or item, and 16-byte vectors its first read takes
        auto where_of = [&](uint32_t k, int64_t tn, uint32_t* n4_first) __attribute__((always_inline)) -> uint64_t {
            if constexpr (SPLIT) {
                *n4_first = lane_value(my_comp, k) ? (lane_value(my_pw, k) + 3) >> 2 : n4_raw;
                return (uint64_t)tn * geo.L;
            }
            if (!packed) {
                *n4_first = n4_spec;
                return (uint64_t)tn * geo.L;
            }
            *n4_first = min(n4_spec, lane_value(my_len, k) >> 4);
            return ((uint64_t)lane_value(o_hi, k) << 32) | lane_value(o_lo, k);
        };
        auto issue = [&](uint32_t k) __attribute__((always_inline)) {
            const int64_t tn = tensor_of2(k);
            if (tn < 0) return;
            uint32_t n4_first;
            const u32x4* s4 = reinterpret_cast<const u32x4*>(slots + where_of(k, tn, &n4_first));
#pragma unroll
            for (int r = 0; r < kSt; ++r) {
                const uint32_t i = lane + (uint32_t)r * kWave;
                if (i < n4_first) st[r] = __builtin_nontemporal_load(s4 + i);
            }
        };

        issue(0);
        if constexpr (!SPLIT) {
            if (lane < cnt && my_tensor >= 0)
                my_comp = (bitmask[(uint64_t)my_tensor >> 5] >> ((uint64_t)my_tensor & 31)) & 1u;
        }
        if (ballot(bad_id)) latch_error(err, kErrRange);
        if (ballot(bad_item || bad_rec)) latch_error(err, kErrCorrupt);
        for (uint32_t k = 0; k < cnt; ++k) {
            const int64_t tn = tensor_of2(k);
            const uint32_t comp = lane_value(my_comp, k);
            const uint64_t oi = first + (base + k) * stride;
            uint32_t* out = reinterpret_cast<uint32_t*>(dst + oi * geo.L);
            uint32_t n4_first = 0, len = 0;
            const uint8_t* item = nullptr;
            if (tn >= 0) {
                item = slots + where_of(k, tn, &n4_first);
                len = packed ? lane_value(my_len, k) : (uint32_t)geo.L;
                if (comp) {
#pragma unroll
                    for (int r = 0; r < kSt; ++r) {
                        const uint32_t i = lane + (uint32_t)r * kWave;
                        if (i < n4_first) reinterpret_cast<u32x4*>(buf)[i] = st[r];
                    }
                } else if (len < geo.L) {
                    latch_error(err, kErrCorrupt);  // a raw item shorter than the tensor
                } else {
                    // raw slot: the prefix from registers, the rest copied
#pragma unroll
                    for (int r = 0; r < kSt; ++r) {
                        const uint32_t i = lane + (uint32_t)r * kWave;
                        if (i < n4_first) __builtin_nontemporal_store(st[r], reinterpret_cast<u32x4*>(out) + i);
                    }
                    if (n4_first < n4_raw)
                        copy_words(reinterpret_cast<const uint32_t*>(item), out, 4ull * n4_first,
                                   4u * (n4_raw - n4_first), true);
                }
            }
            if (k + 1 < cnt) issue(k + 1);
            if (tn < 0 || !comp) continue;

            if constexpr (SPLIT) {
                // header words back in LDS after the payload area, then rebuild
                uint32_t* hdr = buf + nwords + 4;
                const uint32_t H0 = lane_value(h0, k), H1 = lane_value(h1, k), H2 = lane_value(h2, k),
                               H3 = lane_value(h3, k);
                if (lane < hw) hdr[lane] = lane == 0 ? H0 : lane == 1 ? H1 : lane == 2 ? H2 : H3;
                if (lane == 0) buf[4 * n4_first] = 0;
                __builtin_amdgcn_wave_barrier();
                if (UNI)
                    decode_tile<RUNS, MW4, kTileMode>(tu, geo, hdr, buf, 0, 0, nwords, out, true);
                else
                    decode_tile<RUNS, MW4, kTileMode>(ta, geo, hdr, buf, 0, 0, nwords, out, true);
                __builtin_amdgcn_wave_barrier();
                continue;
            }
            __builtin_amdgcn_wave_barrier();
            if (packed || 4 * n4_first >= nwords) {
                // The whole slot (or the whole packed item, whose length the
                // offsets give) is in LDS already, so the record length is
                // needed only to validate it: the rebuild returns the payload
                // bits it consumed (its reads stay inside this wave's buffer,
                // sized hw + n_words + 1 words or more, even for a corrupt
                // header whose chunks all claim to be verbatim), and only the
                // last header word can hold padding bits.
                const uint32_t valid = (uint32_t)(geo.n_chunks - 32ull * (hw - 1));
                const bool bad_pad = valid < 32 && (buf[hw - 1] >> valid) != 0;
                if (lane == 0) buf[4 * n4_first] = 0;
                __builtin_amdgcn_wave_barrier();
                uint32_t pbits;
                if (UNI)
                    pbits = decode_tile<RUNS, MW4, kTileMode>(tu, geo, buf, buf + hw, 0, 0, nwords, out, true);
                else
                    pbits = decode_tile<RUNS, MW4, kTileMode>(ta, geo, buf, buf + hw, 0, 0, nwords, out, true);
                const uint64_t words = hw + (pbits + 31) / 32;
                if (bad_pad || 4ull * words >= geo.L || 4ull * words > len) latch_error(err, kErrCorrupt);
                __builtin_amdgcn_wave_barrier();
                continue;
            }
            bool bad_pad;
            const uint32_t rem = header_removed_bits(planes, geo, buf, 0, hw, &bad_pad);
            const uint64_t R = 32ull * hw + 32ull * nwords - rem;
            const uint32_t words = (uint32_t)((R + 31) / 32);
            if (bad_pad || 4ull * words >= geo.L || 4ull * words > len) {
                latch_error(err, kErrCorrupt);
                continue;
            }
            uint32_t have = 4 * n4_first;
            if (words > have) {
                load_exact_to_lds(reinterpret_cast<const uint32_t*>(item), have, words, buf + have);
                have = words;
            }
            if (lane == 0) buf[have] = 0;
            __builtin_amdgcn_wave_barrier();
            if (UNI)
                decode_tile<RUNS, MW4, kTileMode>(tu, geo, buf, buf + hw, 0, 0, nwords, out, true);
            else
                decode_tile<RUNS, MW4, kTileMode>(ta, geo, buf, buf + hw, 0, 0, nwords, out, true);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// Start bits of the groups of tiles without look-back, for records already in
// HBM, where a second read of the header words (1/W of the tensor's bits)
// costs less than a look-back wait per group.  k_group_bits: a wave takes
// kGroupsPerWave groups and writes each group's payload bits (its chunks'
// widths from its participation bits and the bit planes); k_group_scan: one
// workgroup per tensor turns them into exclusive start bits, the header words
// first.
// Groups of raw tensors or bad ids get 0; the decode reports those itself.
// ---------------------------------------------------------------------------
constexpr uint32_t kGroupsPerWave = 4;

template <uint32_t TPG, uint32_t TW>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void k_group_bits(Tables t, Geo geo,
                                                                       const uint8_t* __restrict__ slots,
                                                                       uint64_t n_slots,
                                                                       const uint32_t* __restrict__ bitmask,
                                                                       const int64_t* __restrict__ ids,
                                                                       uint64_t n_out, uint64_t* bits) {
    // The bit planes of one entry (the same for every header word) are kept
    // in registers; more entries go to LDS when they fit (every header word
    // reads np of them).
    __shared__ uint32_t lds_planes[kMaxLdsPlaneBytes / 4];
    const uint32_t n_plane_words = (geo.Pc / geo.G) * (uint32_t)kPlanes;
    const bool one_entry = n_plane_words == (uint32_t)kPlanes;
    const bool staged = !one_entry && 4ull * n_plane_words <= kMaxLdsPlaneBytes;
    if (staged) {
        for (uint32_t i = threadIdx.x; i < n_plane_words; i += blockDim.x) lds_planes[i] = t.planes[i];
        __syncthreads();
    }
    const uint32_t lane = lane_id();
    const uint64_t gpt = tile_groups(geo.tiles_per_tensor, TPG);
    const uint64_t first = ((uint64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x / kWave)) * kGroupsPerWave;
    // A group has at most TPG * TW / 32 header words (one chunk per word at
    // most): kU per lane, read for all kGroupsPerWave groups before any is
    // summed.  Word u of a lane is header word j(u) of its group (16-byte
    // vectors when the slots are aligned and a lane's words make whole
    // vectors).
    constexpr uint32_t kU = (TPG * TW / 32 + kWave - 1) / kWave;
    static_assert(kU >= 1, "a group has at least one tile of 64 header words at most");
    const bool vec = (kU % 4 == 0) && geo.aligned16 != 0;  // whole vectors per lane
    auto j_of = [&](uint32_t u) __attribute__((always_inline)) {
        return vec ? 4 * lane + 4 * kWave * (u / 4) + (u & 3) : lane + kWave * u;
    };
    const uint64_t total = n_out * gpt;
    // the tensor of each group, then its bitmask bit, then its header words,
    // each step for all groups before the next
    int64_t tensor[kGroupsPerWave];
#pragma unroll
    for (uint32_t k = 0; k < kGroupsPerWave; ++k) {
        const uint64_t oi = min(first + k, total - 1) / gpt;
        tensor[k] = ids ? (int64_t)uniform64((uint64_t)ids[oi]) : (int64_t)oi;
    }
    bool live[kGroupsPerWave];
#pragma unroll
    for (uint32_t k = 0; k < kGroupsPerWave; ++k) {
        live[k] = first + k < total && tensor[k] >= 0 && (uint64_t)tensor[k] < n_slots;
        if (live[k]) live[k] = (uniform(bitmask[(uint64_t)tensor[k] >> 5]) >> ((uint64_t)tensor[k] & 31)) & 1u;
    }
    uint32_t h[kGroupsPerWave][kU];
    uint64_t hw0[kGroupsPerWave], span[kGroupsPerWave];
    uint32_t hw_g[kGroupsPerWave];
#pragma unroll
    for (uint32_t k = 0; k < kGroupsPerWave; ++k) {
        const uint64_t group = min(first + k, total - 1);
        const uint64_t w0 = (group % gpt) * TPG * geo.tile_words;
        span[k] = min(w0 + (uint64_t)TPG * geo.tile_words, geo.n_words) - w0;
        hw0[k] = (w0 >> geo.log2g) >> 5;
        hw_g[k] = (uint32_t)(((span[k] >> geo.log2g) + 31) / 32);
        if (!live[k]) continue;
        const uint32_t* hs = reinterpret_cast<const uint32_t*>(slots + (uint64_t)tensor[k] * geo.L) + hw0[k];
        // loads past the group's header words read its first word again
        if (vec) {
#pragma unroll
            for (uint32_t i = 0; i < kU / 4; ++i) {
                const uint32_t jv = j_of(4 * i) < hw_g[k] ? j_of(4 * i) : 0u;
                const u32x4 x = *reinterpret_cast<const u32x4*>(hs + jv);
#pragma unroll
                for (uint32_t c = 0; c < 4; ++c) h[k][4 * i + c] = x[c];
            }
        } else {
#pragma unroll
            for (uint32_t u = 0; u < kU; ++u) h[k][u] = hs[j_of(u) < hw_g[k] ? j_of(u) : 0u];
        }
    }
    // removed(gj, h): removed bits of header word gj holding h
    auto sum_groups = [&](auto removed) __attribute__((always_inline)) {
#pragma unroll
        for (uint32_t k = 0; k < kGroupsPerWave; ++k) {
            if (first + k >= total) break;
            uint32_t rem = 0;
            if (live[k]) {
#pragma unroll
                for (uint32_t u = 0; u < kU; ++u) {
                    const uint64_t gj = hw0[k] + j_of(u);
                    uint32_t hw = j_of(u) < hw_g[k] ? h[k][u] : 0u;
                    if (gj == geo.hdr_words - 1) {  // bits past the last chunk count nothing
                        const uint32_t valid = (uint32_t)(geo.n_chunks - 32ull * gj);
                        if (valid < 32) hw &= (1u << valid) - 1u;
                    }
                    rem += removed(gj, hw);
                }
            }
            const uint32_t tot = wave_sum(rem);
            if (lane == 0) bits[first + k] = live[k] ? 32 * span[k] - tot : 0;
        }
    };
    if (geo.Pc == 1) {
        // one chunk per period: every chunk removes the same k bits
        sum_groups([&](uint64_t, uint32_t hw) __attribute__((always_inline)) {
            return (uint32_t)__builtin_popcount(hw) * geo.k1;
        });
    } else if (one_entry) {
        // planes past np are zero
        uint32_t pl[kPlanes];
#pragma unroll
        for (int q = 0; q < kPlanes; ++q) pl[q] = t.planes[q];
        sum_groups([&](uint64_t, uint32_t hw) __attribute__((always_inline)) {
            uint32_t r = 0;
#pragma unroll
            for (int q = 0; q < kPlanes; ++q) r += (uint32_t)__builtin_popcount(hw & pl[q]) << q;
            return r;
        });
    } else if (staged) {
        sum_groups([&](uint64_t gj, uint32_t hw) __attribute__((always_inline)) {
            return removed_bits_pl(lds_planes, geo, gj, hw);
        });
    } else {
        sum_groups([&](uint64_t gj, uint32_t hw) __attribute__((always_inline)) {
            return removed_bits_pl(t.planes, geo, gj, hw);
        });
    }
}

__global__ __launch_bounds__(256) void k_group_scan(uint64_t gpt, uint64_t base, uint64_t* bits) {
    __shared__ uint64_t part[256];
    uint64_t* v = bits + (uint64_t)blockIdx.x * gpt;
    const uint32_t tid = threadIdx.x;
    const uint64_t per = (gpt + 255) / 256;
    const uint64_t lo = min(tid * per, gpt), hi = min(lo + per, gpt);
    uint64_t sum = 0;
    for (uint64_t i = lo; i < hi; ++i) sum += v[i];
    part[tid] = sum;
    __syncthreads();
    // inclusive scan of the 256 partial sums (Hillis-Steele)
    for (uint32_t d = 1; d < 256; d <<= 1) {
        const uint64_t add = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    uint64_t run = base + part[tid] - sum;
    for (uint64_t i = lo; i < hi; ++i) {
        const uint64_t x = v[i];
        v[i] = run;
        run += x;
    }
}

hipError_t launch_group_scan(uint64_t n_tensors, uint64_t gpt, uint64_t base, uint64_t* bits, hipStream_t s) {
    // one workgroup per tensor, at most 2^20 workgroups per launch
    constexpr uint64_t kMaxBlocks = 1ull << 20;
    for (uint64_t t0 = 0; t0 < n_tensors; t0 += kMaxBlocks) {
        const uint64_t nb = min(n_tensors - t0, kMaxBlocks);
        hipLaunchKernelGGL(k_group_scan, dim3((uint32_t)nb), dim3(256), 0, s, gpt, base, bits + t0 * gpt);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Tensors longer than one tile.  A wave takes a group of up to
// TPG consecutive tiles of one tensor and reads the header
// words of its whole group at once.  With `starts` (from k_group_bits and
// k_group_scan) the group's start bit is read from there and groups follow
// the block index.  Otherwise it is found by decoupled look-back: thread 0
// of a workgroup takes one ticket for its waves, whose groups follow each
// other, so groups are numbered in the order their workgroups started and a
// group waits only on groups that are resident or done; the wave publishes
// its group's payload bits and sums those of earlier groups of the tensor
// (one atomic and one look-back per group instead of per tile).  It then
// reads and rebuilds its tiles one after another (each tile's start bit is
// the group's plus the earlier tiles' bits, from their header words).
// ---------------------------------------------------------------------------
template <int RUNS, bool UNI, uint32_t TPG, uint32_t TW>
__global__ __launch_bounds__(kWave * kGroupWaves) void k_decode_groups(Tables t, Geo geo, const uint8_t* __restrict__ slots,
                                                       uint64_t n_slots, const uint32_t* __restrict__ bitmask,
                                                       const int64_t* __restrict__ ids, uint64_t n_out,
                                                       uint8_t* __restrict__ dst, uint32_t* err, LookBack lb,
                                                       const uint64_t* __restrict__ starts, uint32_t lds_words) {
    extern __shared__ uint32_t smem[];
    __shared__ uint32_t block_ticket;
    const uint32_t lane = lane_id();
    const uint32_t wib = uniform(threadIdx.x / kWave);
    uint32_t* lds = smem + wib * lds_words;
    if (!starts) {
        if (threadIdx.x == 0) block_ticket = atomicAdd(lb.ticket, 1u);
        __syncthreads();
    }
    const uint64_t group = (uint64_t)(starts ? blockIdx.x : uniform(block_ticket)) * kGroupWaves + wib;
    const uint64_t tpt = geo.tiles_per_tensor;
    const uint64_t gpt = tile_groups(tpt, TPG);
    if (group >= n_out * gpt) return;
    const uint64_t oi = group / gpt;
    const uint64_t lg = group - oi * gpt;
    const uint64_t t0 = lg * TPG;
    const uint32_t n_tiles = (uint32_t)min((uint64_t)TPG, tpt - t0);

    // every group of a tensor sees the same id and bitmask bit, so a bad id
    // or a raw tensor ends all of them before the look-back
    const int64_t tensor = ids ? (int64_t)uniform64((uint64_t)ids[oi]) : (int64_t)oi;
    if (tensor < 0 || (uint64_t)tensor >= n_slots) {
        latch_error(err, kErrRange);
        return;
    }
    const uint32_t* src = reinterpret_cast<const uint32_t*>(slots + (uint64_t)tensor * geo.L);
    uint32_t* out = reinterpret_cast<uint32_t*>(dst + oi * geo.L);
    const uint32_t tw = geo.tile_words;
    const uint64_t w0 = t0 * tw;
    const uint64_t wend = min(w0 + (uint64_t)n_tiles * tw, geo.n_words);
    const bool vec = geo.aligned16 != 0;
    const bool comp = (uniform(bitmask[(uint64_t)tensor >> 5]) >> ((uint64_t)tensor & 31)) & 1u;
    if (!comp) {
        copy_words(src, out, w0, (uint32_t)(wend - w0), vec);
        return;
    }
    TabArrays ta{t.b, t.kd, t.dx, t.r, geo.Mw};
    TabUniform<RUNS> tu;
    if (UNI) tu = load_uniform<RUNS>(t, geo.Mw);

    // header words of the group (a tile's chunks start on a header word)
    const uint32_t hw_tile = (tw >> geo.log2g) / 32;
    const uint64_t hw0 = (w0 >> geo.log2g) >> 5;
    const uint32_t hw_g = (uint32_t)((((wend - w0) >> geo.log2g) + 31) / 32);
    uint32_t* hdr = lds;
    uint32_t* pay = lds + TPG * (TW / 32);
    for (uint32_t j = lane; j < hw_g; j += kWave) hdr[j] = src[hw0 + j];
    __builtin_amdgcn_wave_barrier();
    uint32_t agg[TPG];
    uint64_t agg_all = 0;
    bool bad_pad = false;
#pragma unroll
    for (uint32_t r = 0; r < TPG; ++r) {
        agg[r] = 0;
        if (r < n_tiles) {
            const uint32_t nw = (uint32_t)min((uint64_t)tw, wend - (w0 + (uint64_t)r * tw));
            const uint32_t hw_t = ((nw >> geo.log2g) + 31) / 32;
            bool bad;
            const uint32_t rem = header_removed_bits(t.planes, geo, hdr + r * hw_tile, hw0 + r * hw_tile, hw_t, &bad);
            bad_pad = bad_pad || bad;
            agg[r] = 32u * nw - rem;
            agg_all += agg[r];
        }
    }
    const uint64_t S = starts ? uniform64(starts[group])
                              : lookback_exclusive(lb.status, oi * gpt, lg, agg_all, 32ull * geo.hdr_words, lb.epoch,
                                                   err);
    const uint64_t E = S + agg_all;
    const bool last = lg == gpt - 1;
    if (bad_pad || E > 8ull * geo.L || (last && 4 * ((E + 31) / 32) >= geo.L)) {
        latch_error(err, kErrCorrupt);
        return;
    }
    // payload words [a, b) of tile r, whose fields start at bit St (16-byte
    // rounded when vec)
    auto tile_range = [&](uint64_t St, uint32_t r, uint64_t* a, uint64_t* b) __attribute__((always_inline)) {
        *a = St >> 5;
        *b = (St + agg[r] + 31) >> 5;
        if (vec) {
            *a &= ~3ull;
            *b = (*b + 3) & ~3ull;
        }
        *b = min(*b, geo.n_words);
    };
    // Records in HBM, with 16-byte vectors: the next tile's payload (at most
    // 2,048 + 8 words, so kPre vectors per lane) is read into registers while
    // the current tile is rebuilt from LDS (32 llm_bf16 layers from HBM:
    // 1,355 -> 1,172 us, and 1,100 us with the buffer loads below).  Over the
    // host link the reads in flight of many waves already fill the link, and
    // this prefetch measured slower (1,252 -> 1,267 us per layer alone), so
    // there each tile is read when due.
    const bool pipelined = vec && geo.src_in_hbm;
    constexpr uint32_t kPre = (TW + 8 + 4 * kWave - 1) / (4 * kWave);
    u32x4 pre[kPre];
    // kPre buffer loads per lane whose range is payload words [a, b): vectors
    // past it return zero without touching memory, so every tile issues the
    // same number of loads whatever its length.  Word 3 of the descriptor is
    // the gfx9 raw-buffer format (32-bit data, no swizzle); cache policy 2 is
    // the non-temporal hint.
    auto issue = [&](uint64_t a, uint64_t b) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(src + uniform64(a)), (short)0, (int)uniform((uint32_t)(4 * (b - a))), 0x00020000);
#pragma unroll
        for (uint32_t i = 0; i < kPre; ++i)
            pre[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(16 * (lane + i * kWave)), 0, 2);
    };
    // the loaded words [a, b) into pay, and the zero word after them
    auto stage = [&](uint64_t a, uint64_t b) __attribute__((always_inline)) {
        const uint32_t n4 = (uint32_t)((b - a) >> 2);
#pragma unroll
        for (uint32_t i = 0; i < kPre; ++i)
            if (lane + i * kWave < n4) reinterpret_cast<u32x4*>(pay)[lane + i * kWave] = pre[i];
        if (lane == 0) pay[b - a] = 0;
    };
    uint64_t St = S;
    // the rebuild of tile r from pay (any length)
    auto rebuild = [&](uint32_t r, uint64_t a) __attribute__((always_inline)) {
        const uint64_t wt = w0 + (uint64_t)r * tw;
        const uint32_t nw = (uint32_t)min((uint64_t)tw, wend - wt);
        if (UNI)
            decode_tile<RUNS, false, kTileMultiStep>(tu, geo, hdr + r * hw_tile, pay, (uint32_t)(St - 32 * a), wt, nw, out,
                                           vec && (wt & 3) == 0);
        else
            decode_tile<RUNS, false, kTileMultiStep>(ta, geo, hdr + r * hw_tile, pay, (uint32_t)(St - 32 * a), wt, nw, out,
                                           vec && (wt & 3) == 0);
    };
    const uint32_t n_full = (uint32_t)((wend - w0) / tw);
    if (pipelined && n_full > 0 && tw == TW) {
        // Each iteration rebuilds full tile r (TW / 256 unrolled
        // steps, one store each), then writes tile r + 1's prefetched vectors
        // to LDS and issues tile r + 2's loads.  The loop is entered with
        // tile 0 staged and tile 1's loads in flight, the same pattern its
        // back edge carries, so before each LDS write the compiler waits for
        // that vector's load alone and leaves the tile's stores in flight.
        // (A second register buffer, two tiles ahead, measured no faster.)
        uint64_t a, b;
        tile_range(St, 0, &a, &b);
        issue(a, b);
        stage(a, b);
        if (n_tiles > 1) {
            uint64_t an, bn;
            tile_range(St + agg[0], 1, &an, &bn);
            issue(an, bn);
        }
        for (uint32_t r = 0; r < n_full; ++r) {
            __builtin_amdgcn_wave_barrier();  // the staged words are written
            if (UNI)
                decode_full_tile<RUNS, TW>(tu, geo, hdr + r * hw_tile, pay, (uint32_t)(St - 32 * a), w0 + (uint64_t)r * tw,
                                       out);
            else
                decode_full_tile<RUNS, TW>(ta, geo, hdr + r * hw_tile, pay, (uint32_t)(St - 32 * a), w0 + (uint64_t)r * tw,
                                       out);
            St += agg[r];
            if (r + 1 < n_tiles) {
                tile_range(St, r + 1, &a, &b);
                __builtin_amdgcn_wave_barrier();  // this tile's reads of pay are done
                stage(a, b);
                if (r + 2 < n_tiles) {
                    uint64_t an, bn;
                    tile_range(St + agg[r + 1], r + 2, &an, &bn);
                    issue(an, bn);
                }
            }
        }
        if (n_full < n_tiles) {  // the tensor's ragged last tile, staged by the loop
            __builtin_amdgcn_wave_barrier();
            rebuild(n_full, a);
        }
        return;
    }
    for (uint32_t r = 0; r < n_tiles; ++r) {
        const uint64_t Et = St + agg[r];
        uint64_t a, b;
        tile_range(St, r, &a, &b);
        __builtin_amdgcn_wave_barrier();  // the previous tile's reads of pay are done
        if (pipelined) {  // a single ragged tile
            issue(a, b);
            stage(a, b);
        } else {
            load_words_to_lds(src, a, b, pay, vec);
            if (lane == 0) pay[b - a] = 0;
        }
        __builtin_amdgcn_wave_barrier();
        rebuild(r, a);
        St = Et;
    }
}

// ---------------------------------------------------------------------------
// Single-tile tensors the persistent kernel does not take: slots or output
// not 16-byte aligned, or tables too large for LDS.  One wave per tensor,
// tables read from global memory; the record's first read, then (once the
// header gives its length) the rest.
// ---------------------------------------------------------------------------
template <int RUNS, bool UNI>
__global__ __launch_bounds__(256) void k_decode_tiles(Tables t, Geo geo, const uint8_t* __restrict__ slots,
                                                      uint64_t n_slots, const uint32_t* __restrict__ bitmask,
                                                      const int64_t* __restrict__ ids, uint64_t n_out,
                                                      uint8_t* __restrict__ dst, uint32_t* err, uint32_t lds_words) {
    extern __shared__ uint32_t smem[];
    const uint32_t lane = lane_id();
    uint32_t* lds = smem + (threadIdx.x / kWave) * lds_words;
    const uint64_t oi = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (oi >= n_out) return;
    const int64_t tensor = ids ? (int64_t)uniform64((uint64_t)ids[oi]) : (int64_t)oi;
    if (tensor < 0 || (uint64_t)tensor >= n_slots) {
        latch_error(err, kErrRange);
        return;
    }
    const uint32_t* src = reinterpret_cast<const uint32_t*>(slots + (uint64_t)tensor * geo.L);
    uint32_t* out = reinterpret_cast<uint32_t*>(dst + oi * geo.L);
    const uint32_t nw = (uint32_t)geo.n_words;
    const bool vec = geo.aligned16 != 0;
    const bool comp = (uniform(bitmask[(uint64_t)tensor >> 5]) >> ((uint64_t)tensor & 31)) & 1u;
    if (!comp) {
        copy_words(src, out, 0, nw, vec);
        return;
    }
    TabArrays ta{t.b, t.kd, t.dx, t.r, geo.Mw};
    TabUniform<RUNS> tu;
    if (UNI) tu = load_uniform<RUNS>(t, geo.Mw);
    const uint32_t hw = (uint32_t)geo.hdr_words;
    uint32_t have = geo.spec_words;
    load_words_to_lds(src, 0, have, lds, vec);
    __builtin_amdgcn_wave_barrier();
    bool bad_pad;
    const uint32_t rem = header_removed_bits(t.planes, geo, lds, 0, hw, &bad_pad);
    const uint64_t R = 32ull * hw + 32ull * geo.n_words - rem;
    const uint64_t words = (R + 31) / 32;
    if (bad_pad || 4 * words >= geo.L) {
        latch_error(err, kErrCorrupt);
        return;
    }
    if (words > have) {
        const uint32_t need = vec ? (uint32_t)((words + 3) & ~3ull) : (uint32_t)words;
        const uint32_t upto = min(need, nw);
        load_words_to_lds(src, have, upto, lds + have, vec);
        have = upto;
    }
    if (lane == 0) lds[have] = 0;
    __builtin_amdgcn_wave_barrier();
    if (UNI)
        decode_tile<RUNS, false, kTileOneStep>(tu, geo, lds, lds + hw, 0, 0, nw, out, vec);
    else
        decode_tile<RUNS, false, kTileOneStep>(ta, geo, lds, lds + hw, 0, 0, nw, out, vec);
}

// ---------------------------------------------------------------------------
// Short launches from GPU memory: tensors of at most 1 KiB (one 16-byte
// vector per lane holds the whole slot or item) and at most a few rows per
// CU.  A wave takes RPW output rows, four waves to a workgroup, nothing
// staged: the rows' records, their bitmask words and the table entries of
// the lanes' positions (or the few wave-uniform words of uniform metadata)
// are loaded at once, straight into registers, so the rows cost one round
// trip to memory after their ids (and, in the packed layout, their item
// spans).  A fixed slot is read whole; the persistent kernel, which stages
// the tables per workgroup and reads only the record, keeps the longer
// launches, where its waves decode several rows each.
// ---------------------------------------------------------------------------

// Table entries of one lane's NW consecutive positions (Mw a multiple of 4),
// loaded once into registers; the accessors decode_step / decode_step2 use.
template <int RUNS, int NW>
struct TabRegs {
    static_assert(RUNS <= 3, "run shifts past the third live in the dx rows");
    using V = std::conditional_t<NW == 4, u32x4, u32x2>;
    V kd, b;
    V r[RUNS > 0 ? RUNS : 1];
    __device__ __forceinline__ void load(const Tables& t, uint32_t Mw, uint32_t pos0) {
        kd = *reinterpret_cast<const V*>(t.kd + pos0);
        b = *reinterpret_cast<const V*>(t.b + pos0);
#pragma unroll
        for (int j = 0; j < RUNS; ++j) r[j] = *reinterpret_cast<const V*>(t.r + (uint32_t)j * Mw + pos0);
    }
    __device__ __forceinline__ V kdw4(uint32_t) const { return kd; }
    __device__ __forceinline__ V bw4(uint32_t) const { return b; }
    __device__ __forceinline__ V rw4(int j, uint32_t) const { return r[j]; }
    __device__ __forceinline__ V kdw2(uint32_t) const { return kd; }
    __device__ __forceinline__ V bw2(uint32_t) const { return b; }
    __device__ __forceinline__ V rw2(int j, uint32_t) const { return r[j]; }
    __device__ __forceinline__ uint32_t dw(int j, uint32_t, uint32_t kdv) const { return kdv >> (8 * (j + 1)); }
};

// NW: words per lane of the rebuild (2 for tensors of at most 128 words, else
// 4).  PACKED: items at items.offsets (else fixed slots of L bytes).  RPW:
// rows per wave, whose loads are all in flight before the first is rebuilt.
template <int RUNS, bool UNI, int NW, bool PACKED, int RPW>
__global__ __launch_bounds__(256) void k_decode_rows(Tables t, Geo geo, const uint8_t* __restrict__ base,
                                                     uint64_t n_slots, const uint32_t* __restrict__ bitmask,
                                                     const int64_t* __restrict__ ids, uint64_t n_out,
                                                     uint8_t* __restrict__ dst, uint32_t* err, uint32_t buf_words,
                                                     Items items) {
    extern __shared__ uint32_t smem[];
    const uint32_t lane = lane_id();
    const uint32_t wib = uniform(threadIdx.x / kWave);
    const uint64_t oi0 = ((uint64_t)blockIdx.x * (blockDim.x / kWave) + wib) * RPW;
    if (oi0 >= n_out) return;
    if (n_slots == 0) {
        latch_error(err, kErrRange);
        return;
    }
    // Each round of loads (ids; item spans and bitmask words; records) is
    // issued for all the wave's rows before any of them is waited for.  A row
    // that is past the launch or has a bad id or span keeps id 0 and reads
    // nothing.
    int64_t raw_id[RPW];
    static_for<RPW>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        raw_id[r] = ids ? ids[min(oi0 + r, n_out - 1)] : (int64_t)(oi0 + r);
    });
    int64_t id[RPW];
    bool live[RPW];
    static_for<RPW>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const int64_t v = (int64_t)uniform64((uint64_t)raw_id[r]);
        const bool in_launch = oi0 + r < n_out;
        live[r] = in_launch && v >= 0 && (uint64_t)v < n_slots;
        if (in_launch && !live[r]) latch_error(err, kErrRange);
        id[r] = live[r] ? v : 0;
    });
    uint64_t a[RPW], b[RPW];
    uint32_t bw[RPW];
    static_for<RPW>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        if constexpr (PACKED) {
            a[r] = items.offsets[id[r]];
            b[r] = items.offsets[id[r] + 1];
        } else {
            a[r] = (uint64_t)id[r] * geo.L;
            b[r] = a[r] + geo.L;
        }
        bw[r] = bitmask[(uint64_t)id[r] >> 5];
    });
    uint32_t len[RPW];
    u32x4 v[RPW];
    static_for<RPW>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        a[r] = uniform64(a[r]);
        b[r] = uniform64(b[r]);
        if (PACKED && live[r] &&
            (b[r] < a[r] || b[r] > items.bytes || ((a[r] | b[r]) & 15) || b[r] - a[r] > ((geo.L + 15) & ~15ull))) {
            latch_error(err, kErrCorrupt);
            live[r] = false;
        }
        len[r] = live[r] ? (uint32_t)(b[r] - a[r]) : 0u;
        // range-checked: lanes past the record read zeros
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(base + (live[r] ? a[r] : 0)), (short)0, (int)len[r], 0x00020000);
        v[r] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(16 * lane), 0, 2);
    });
    const uint32_t Mw = geo.Mw;
    TabUniform<RUNS> tu;
    TabRegs<UNI ? 0 : RUNS, NW> tr;
    if constexpr (UNI) {
        tu = load_uniform<RUNS>(t, Mw);
    } else {
        // a period of at least a step's words needs no wrap (and no division)
        const uint32_t p0 = (uint32_t)NW * lane;
        if (Mw >= (uint32_t)NW * kWave)
            tr.load(t, Mw, p0);
        else
            tr.load(t, Mw, p0 % Mw);
    }
    const uint32_t nwords = (uint32_t)geo.n_words;
    const uint32_t hw = (uint32_t)geo.hdr_words;
    uint32_t* buf = smem + wib * buf_words;
    static_for<RPW>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        if (!live[r]) return;
        const uint32_t comp = (uniform(bw[r]) >> ((uint64_t)id[r] & 31)) & 1u;
        uint32_t* out = reinterpret_cast<uint32_t*>(dst + (oi0 + r) * geo.L);
        if (!comp) {
            // a raw slot or item holds the tensor's bytes
            if (len[r] < geo.L)
                latch_error(err, kErrCorrupt);
            else if (lane < (nwords >> 2))
                __builtin_nontemporal_store(v[r], reinterpret_cast<u32x4*>(out) + lane);
            return;
        }
        const uint32_t n4 = len[r] >> 4;
        if (lane < n4) reinterpret_cast<u32x4*>(buf)[lane] = v[r];
        if (lane == 0) buf[4 * n4] = 0;
        __builtin_amdgcn_wave_barrier();
        // The whole record is in LDS, so its length only validates it: the
        // rebuild returns the payload bits it consumed, and its reads stay
        // inside the buffer (hw + n_words + 1 words or more) whatever the
        // header says.
        const uint32_t valid = (uint32_t)(geo.n_chunks - 32ull * (hw - 1));
        const bool bad_pad = valid < 32 && (buf[hw - 1] >> valid) != 0;
        constexpr int kMode = NW == 2 ? kTileHalfStep : kTileOneStep;
        uint32_t pbits;
        if constexpr (UNI)
            pbits = decode_tile<RUNS, true, kMode>(tu, geo, buf, buf + hw, 0, 0, nwords, out, true);
        else
            pbits = decode_tile<RUNS, true, kMode>(tr, geo, buf, buf + hw, 0, 0, nwords, out, true);
        // tensors of at most 1 KiB: 32-bit compares
        const uint32_t words = hw + (pbits + 31) / 32;
        if (bad_pad || 4 * words >= (uint32_t)geo.L || 4 * words > len[r]) latch_error(err, kErrCorrupt);
        __builtin_amdgcn_wave_barrier();
    });
}

// ---------------------------------------------------------------------------
// Launch.
// ---------------------------------------------------------------------------
static uint32_t runs_bucket(uint32_t runs) {
    if (runs <= 4) return runs;
    if (runs <= 8) return 8;
    return 16;
}

// LDS k_decode_small shares per workgroup (tables, planes) and needs per
// wave (record buffer); false when the tables do not fit.
static bool small_lds(const Geo& geo, int runs, bool uni, uint32_t* buf_words, size_t* head, size_t* wave) {
    // a rebuild from a whole slot reads at most word hw + n_words of the
    // buffer (a corrupt header whose chunks all claim to be verbatim), and
    // the header-in-GPU-memory layout puts hw <= 4 words after n_words + 4
    const uint32_t tail = std::max<uint32_t>(8u, (uint32_t)geo.hdr_words + 1);
    *buf_words = ((uint32_t)geo.n_words + tail + 3) & ~3u;
    const uint64_t tab = uni ? 0 : (uint64_t)tab_rows(runs) * geo.Mw * 4;
    const uint64_t planes = (uint64_t)(geo.Pc / geo.G) * kPlanes * 4;
    if (tab > kMaxLdsTableBytes || planes > kMaxLdsPlaneBytes) return false;
    *head = (size_t)(((tab + planes) + 15) & ~15ull);
    *wave = (size_t)*buf_words * 4;
    return true;
}

// Resident waves per SIMD the small-tensor decode keeps at most when the
// stored items are in device memory.  Short tiles give each wave only a few
// tiles per launch, and every wave pays a fixed start (table staging, the
// batch's ids and bitmask words, the first read): with 7 or 8 waves per SIMD,
// 512-byte and 1 KiB rows in HBM decoded 10-25 % slower than with 4 to 6
// (measured on MI355X).  Items read over the host link keep every wave the
// registers allow, since there the reads in flight set the rate.
#ifndef IBP_SMALL_DECODE_WAVES_HBM
#define IBP_SMALL_DECODE_WAVES_HBM 5
#endif
constexpr uint32_t kSmallDecodeWavesPerSimdHbm = IBP_SMALL_DECODE_WAVES_HBM;

template <int RUNS, bool UNI, bool MW4, int S, bool SPLIT>
static hipError_t launch_small_s(const Tables& t, const Geo& geo, const void* slots, uint64_t n_slots,
                                 const uint32_t* bitmask, const int64_t* ids, uint64_t n_out, void* dst,
                                 uint32_t* err, uint32_t cu_count, size_t head, size_t wave, uint32_t buf_words,
                                 const Items& items, const uint32_t* headers, hipStream_t s, bool* launched) {
    const void* fn = reinterpret_cast<const void*>(&k_decode_small<RUNS, UNI, MW4, S, SPLIT>);
    PersistentPlan plan;
    *launched = false;
    if (!plan_persistent(fn, head, wave, cu_count, n_out, &plan, geo.src_in_hbm ? kSmallDecodeWavesPerSimdHbm : 8u,
                         kDecodeItemsPerWave))
        return hipSuccess;
    hipLaunchKernelGGL((k_decode_small<RUNS, UNI, MW4, S, SPLIT>), dim3(plan.blocks), dim3(kWave * plan.wpb),
                       plan.shm, s, t, geo, static_cast<const uint8_t*>(slots), n_slots, bitmask, ids, n_out,
                       static_cast<uint8_t*>(dst), err, buf_words, items, headers);
    *launched = true;
    return hipGetLastError();
}

template <int RUNS, bool UNI>
static hipError_t launch_small(const Tables& t, const Geo& geo, const void* slots, uint64_t n_slots,
                               const uint32_t* bitmask, const int64_t* ids, uint64_t n_out, void* dst,
                               uint32_t* err, uint32_t cu_count, size_t head, size_t wave, uint32_t buf_words,
                               const Items& items, const uint32_t* headers, hipStream_t s, bool* launched) {
    const uint32_t stage = (uint32_t)((geo.n_words + 4 * kWave - 1) / (4 * kWave));
    const bool mw4 = geo.Mw % 4 == 0;
#define IBP_SMALL_X(S, SPLIT)                                                                                  \
    return mw4 ? launch_small_s<RUNS, UNI, true, S, SPLIT>(t, geo, slots, n_slots, bitmask, ids, n_out, dst,   \
                                                           err, cu_count, head, wave, buf_words, items, headers, \
                                                           s, launched)                                          \
               : launch_small_s<RUNS, UNI, false, S, SPLIT>(t, geo, slots, n_slots, bitmask, ids, n_out, dst,  \
                                                            err, cu_count, head, wave, buf_words, items,         \
                                                            headers, s, launched)
#define IBP_SMALL(S)               \
    do {                           \
        if (headers) {             \
            IBP_SMALL_X(S, true);  \
        }                          \
        IBP_SMALL_X(S, false);     \
    } while (0)
    if (geo.n_words <= 2 * kWave) IBP_SMALL(0);
    if (stage <= 1) IBP_SMALL(1);
    if (stage <= 2) IBP_SMALL(2);
    if (stage <= 4) IBP_SMALL(4);
    IBP_SMALL(8);
#undef IBP_SMALL
#undef IBP_SMALL_X
}

// Single-tile tensors of at most 1 KiB in GPU memory, 16-byte aligned, at
// most three runs per position unless the metadata is uniform, and at most
// 128 rows per CU: k_decode_rows.  Measured on MI355X with 1 KiB sparse_gnn
// rows in the packed layout and one row per wave: 1,024 / 8,192 / 32,768 /
// 65,536 / 262,144 ids gathered in 3.4 / 5.9 / 16.9 / 31.1 / 116.4 us,
// against 4.4 / 7.7 / 19.0 / 31.5 / 111.3 us for the persistent kernel, which
// also decodes all 1,048,576 items 5 % faster.  0 sends every call to the
// persistent kernel.
#ifndef IBP_DECODE_ROWS
#define IBP_DECODE_ROWS 1
#endif

static bool decode_rows(const Geo& geo, int runs, bool uni, uint64_t n_out, uint32_t cu_count) {
    return IBP_DECODE_ROWS && geo.src_in_hbm && geo.aligned16 && geo.n_words <= 4 * kWave &&
           (uni || (runs <= 3 && geo.Mw % 4 == 0)) && n_out <= 128ull * cu_count;
}

// Rows per wave of k_decode_rows.  Measured on MI355X (16,384 dense_gnn rows
// of 512 bytes / 8,192-id packed-cache gathers of 1 KiB rows): 1 row 5.9-6.8
// / 6.2-6.4 us, 2 rows 5.5-5.9 / 5.8 us, 4 rows 6.2-6.5 / 6.9 us.
#ifndef IBP_DECODE_ROWS_PER_WAVE
#define IBP_DECODE_ROWS_PER_WAVE 2
#endif
constexpr int kDecodeRowsPerWave = IBP_DECODE_ROWS_PER_WAVE;

template <int RUNS, bool UNI, int NW, bool PACKED>
static hipError_t launch_rows_t(const Tables& t, const Geo& geo, const void* base, uint64_t n_slots,
                                const uint32_t* bitmask, const int64_t* ids, uint64_t n_out, void* dst,
                                uint32_t* err, uint32_t buf_words, const Items& items, hipStream_t s) {
    constexpr uint32_t kRowWaves = 4;
    constexpr uint64_t kRows = kRowWaves * kDecodeRowsPerWave;
    const dim3 grid((uint32_t)((n_out + kRows - 1) / kRows));
    const size_t shm = (size_t)buf_words * 4 * kRowWaves;
    hipLaunchKernelGGL((k_decode_rows<RUNS, UNI, NW, PACKED, kDecodeRowsPerWave>), grid, dim3(kWave * kRowWaves),
                       shm, s, t, geo,
                       static_cast<const uint8_t*>(base), n_slots, bitmask, ids, n_out, static_cast<uint8_t*>(dst),
                       err, buf_words, items);
    return hipGetLastError();
}

template <int RUNS, bool UNI>
static hipError_t launch_rows(const Tables& t, const Geo& geo, const void* base, uint64_t n_slots,
                              const uint32_t* bitmask, const int64_t* ids, uint64_t n_out, void* dst, uint32_t* err,
                              uint32_t buf_words, const Items& items, hipStream_t s) {
    if constexpr (!UNI && RUNS > 3) {
        return hipErrorInvalidValue;
    } else {
        const bool half = geo.n_words <= 2 * kWave;
        if (items.offsets)
            return half ? launch_rows_t<RUNS, UNI, 2, true>(t, geo, base, n_slots, bitmask, ids, n_out, dst, err,
                                                            buf_words, items, s)
                        : launch_rows_t<RUNS, UNI, 4, true>(t, geo, base, n_slots, bitmask, ids, n_out, dst, err,
                                                            buf_words, items, s);
        return half ? launch_rows_t<RUNS, UNI, 2, false>(t, geo, base, n_slots, bitmask, ids, n_out, dst, err,
                                                         buf_words, items, s)
                    : launch_rows_t<RUNS, UNI, 4, false>(t, geo, base, n_slots, bitmask, ids, n_out, dst, err,
                                                         buf_words, items, s);
    }
}

template <int RUNS, bool UNI>
static hipError_t launch_tiles(const Tables& t, const Geo& geo, const void* slots, uint64_t n_slots,
                               const uint32_t* bitmask, const int64_t* ids, uint64_t n_out, void* dst,
                               uint32_t* err, hipStream_t s) {
    // the record (up to the slot) and the zero word after it
    const uint32_t lds_words = (uint32_t)geo.n_words + 8;
    const dim3 grid((uint32_t)((n_out + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(kWave * kWavesPerBlock);
    const size_t shm = (size_t)lds_words * 4 * kWavesPerBlock;
    hipLaunchKernelGGL((k_decode_tiles<RUNS, UNI>), grid, block, shm, s, t, geo, static_cast<const uint8_t*>(slots),
                       n_slots, bitmask, ids, n_out, static_cast<uint8_t*>(dst), err, lds_words);
    return hipGetLastError();
}

// Tensors longer than one tile: one wave per group of tiles; lb holds one
// status word per group (n_out * tile_groups(tiles_per_tensor, TPG)), which the
// look-back uses over the host link and the start bits of the header pass
// and scan use for records in HBM.
template <int RUNS, bool UNI, uint32_t TPG, uint32_t TW>
static hipError_t launch_groups_t(const Tables& t, const Geo& geo, const void* slots, uint64_t n_slots,
                                  const uint32_t* bitmask, const int64_t* ids, uint64_t n_out, void* dst,
                                  uint32_t* err, const LookBack& lb, hipStream_t s) {
    if (geo.tile_words != TW) return hipErrorInvalidValue;
    // header words of a group, then one tile's payload (up to 8 words of
    // 16-byte rounding and the zero word after it)
    const uint32_t lds_words = TPG * (TW / 32) + TW + 8;
    const uint64_t gpt = tile_groups(geo.tiles_per_tensor, TPG);
    const uint64_t groups = n_out * gpt;
    uint64_t* starts = nullptr;
    if (geo.src_in_hbm) {
        // records in HBM: start bits from two short passes over the header
        // words, into the look-back status words
        starts = reinterpret_cast<uint64_t*>(lb.status);
        const uint64_t waves = (groups + kGroupsPerWave - 1) / kGroupsPerWave;
        hipLaunchKernelGGL((k_group_bits<TPG, TW>), dim3((uint32_t)((waves + kWavesPerBlock - 1) / kWavesPerBlock)),
                           dim3(kWave * kWavesPerBlock), 0, s, t, geo, static_cast<const uint8_t*>(slots), n_slots,
                           bitmask, ids, n_out, starts);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_group_scan(n_out, gpt, 32ull * geo.hdr_words, starts, s);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((uint32_t)((groups + kGroupWaves - 1) / kGroupWaves));
    const dim3 block(kWave * kGroupWaves);
    const size_t shm = (size_t)lds_words * 4 * kGroupWaves;
    hipLaunchKernelGGL((k_decode_groups<RUNS, UNI, TPG, TW>), grid, block, shm, s, t, geo,
                       static_cast<const uint8_t*>(slots), n_slots, bitmask, ids, n_out, static_cast<uint8_t*>(dst),
                       err, lb, starts, lds_words);
    return hipGetLastError();
}

// Tensors longer than one tile, with the group and tile sizes of where their
// records are (decode_group_tiles, decode_tile_words).
template <int RUNS, bool UNI>
static hipError_t launch_groups(const Tables& t, const Geo& geo, const void* slots, uint64_t n_slots,
                                const uint32_t* bitmask, const int64_t* ids, uint64_t n_out, void* dst,
                                uint32_t* err, const LookBack& lb, hipStream_t s) {
    if (geo.src_in_hbm)
        return launch_groups_t<RUNS, UNI, decode_group_tiles(true), decode_tile_words(true)>(
            t, geo, slots, n_slots, bitmask, ids, n_out, dst, err, lb, s);
    return launch_groups_t<RUNS, UNI, decode_group_tiles(false), decode_tile_words(false)>(
        t, geo, slots, n_slots, bitmask, ids, n_out, dst, err, lb, s);
}

template <int RUNS, bool UNI>
static hipError_t launch_decode_r(const Tables& t, const Geo& geo, const void* slots, uint64_t n_slots,
                                  const uint32_t* bitmask, const int64_t* ids, uint64_t n_out, void* dst,
                                  uint32_t* err, const LookBack* lb, uint32_t cu_count, hipStream_t s,
                                  const Items& items, const uint32_t* headers) {
    if (geo.tiles_per_tensor > 1) {
        if (items.offsets || headers) return hipErrorInvalidValue;
        return launch_groups<RUNS, UNI>(t, geo, slots, n_slots, bitmask, ids, n_out, dst, err, *lb, s);
    }
    uint32_t buf_words = 0;
    size_t head = 0, wave = 0;
    if (geo.aligned16 && small_lds(geo, RUNS, UNI, &buf_words, &head, &wave)) {
        if (!headers && decode_rows(geo, RUNS, UNI, n_out, cu_count))
            return launch_rows<RUNS, UNI>(t, geo, slots, n_slots, bitmask, ids, n_out, dst, err, buf_words, items,
                                          s);
        bool launched = false;
        const hipError_t e = launch_small<RUNS, UNI>(t, geo, slots, n_slots, bitmask, ids, n_out, dst, err, cu_count,
                                                     head, wave, buf_words, items, headers, s, &launched);
        if (e != hipSuccess || launched) return e;
    }
    // the packed and header-in-GPU-memory layouts run on k_decode_small only
    if (items.offsets || headers) return hipErrorInvalidValue;
    return launch_tiles<RUNS, UNI>(t, geo, slots, n_slots, bitmask, ids, n_out, dst, err, s);
}

bool packed_decode_supported(const Geo& geo, uint32_t runs, bool uniform_meta) {
    uint32_t buf_words = 0;
    size_t head = 0, wave = 0;
    return geo.tiles_per_tensor == 1 && geo.aligned16 &&
           small_lds(geo, (int)runs_bucket(runs), uniform_meta, &buf_words, &head, &wave);
}

hipError_t launch_decode(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta, const void* slots,
                         uint64_t n_slots, const uint32_t* bitmask, const int64_t* ids, uint64_t n_out,
                         void* dst, uint32_t* err, const LookBack* lb, uint32_t cu_count, hipStream_t s,
                         const Items* items, const uint32_t* headers) {
    if (n_out == 0) return hipSuccess;
    const Items it = items ? *items : Items{nullptr, 0};
#define IBP_R(R)                                                                                      \
    return uniform_meta                                                                                \
               ? launch_decode_r<R, true>(t, geo, slots, n_slots, bitmask, ids, n_out, dst, err, lb,    \
                                          cu_count, s, it, headers)                                    \
               : launch_decode_r<R, false>(t, geo, slots, n_slots, bitmask, ids, n_out, dst, err, lb,   \
                                           cu_count, s, it, headers)
    switch (runs_bucket(runs)) {
        case 0: IBP_R(0);
        case 1: IBP_R(1);
        case 2: IBP_R(2);
        case 3: IBP_R(3);
        case 4: IBP_R(4);
        case 8: IBP_R(8);
        default: IBP_R(16);
    }
#undef IBP_R
}

}  // namespace ibp
