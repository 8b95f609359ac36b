// ibp_kernels.hip -- gfx950 kernels of Invariant Bit Packing.
//
// Method: FR summary ("Résumé Technique : Réduire le goulot d'étranglement de
// la mémoire GPU par la compression sans perte pour le ML") and KO summary
// ("Reducing the GPU Memory Bottleneck with Lossless Compression for ML --
// Extended"), section "Algorithme central" / "핵심 알고리즘": step 1 builds
// Mask/Bitval from a sample and a threshold, step 2 tests each chunk against
// Bitval, drops the invariant bits of matching chunks and records one
// participation bit per chunk, step 3 has the lanes of a wave load a
// compressed segment together, scan the chunk sizes for start offsets and put
// the invariant bits back.  Section "Intégration au système": fixed-size
// slots of which only the compressed prefix is read, and a bitmask in GPU
// memory saying which slots are compressed.
//
// Work unit: one wave64 owns one tile (up to 2048 32-bit words of one
// tensor); four independent waves share a workgroup.  A lane handles one
// 32-bit word per step; a chunk of W = 32*g bits spans g adjacent lanes.
// Tensors longer than one tile are cut into tiles that find their start bit
// by decoupled look-back over per-tile status words.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ibp_device.hpp"
#include "ibp_internal.hpp"

namespace ibp {

// ---------------------------------------------------------------------------
// Step 1: preprocessing.
// ---------------------------------------------------------------------------

// Per-position histogram.  The sample is a sequence of observations of Mw
// words; thread g of G (G a multiple of Mw) visits words g, g+G, g+2G, ...,
// which all sit at position g mod Mw, so reads are coalesced.  Bits are
// counted eight at a time in byte lanes (x >> k) & 0x01010101 and flushed
// into 32 counters every 255 observations.
__global__ __launch_bounds__(256) void k_meta_hist(const uint32_t* __restrict__ sample,
                                                   uint64_t n_words, uint32_t Mw, uint64_t G,
                                                   uint32_t* __restrict__ counts) {
    const uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t cnt[32];
#pragma unroll
    for (int b = 0; b < 32; ++b) cnt[b] = 0;
    if (g < G) {
        uint64_t i = g;
        while (i < n_words) {
            uint32_t acc[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = 0;
            for (int r = 0; r < 255 && i < n_words; ++r, i += G) {
                uint32_t x = sample[i];
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] += (x >> k) & 0x01010101u;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int q = 0; q < 4; ++q) cnt[8 * q + k] += (acc[k] >> (8 * q)) & 0xFFu;
        }
    }
    const uint32_t w = (uint32_t)(g % Mw);
    // Lanes of one wave that share a position are folded together first when
    // the period divides the wave; the rest go straight to global atomics.
    if (Mw < (uint32_t)kWave && (kWave % Mw) == 0) {
#pragma unroll
        for (int b = 0; b < 32; ++b)
            for (uint32_t o = Mw; o < (uint32_t)kWave; o <<= 1) cnt[b] += __shfl_xor(cnt[b], (int)o);
        if (lane_id() >= Mw || g >= G) return;
    } else if (g >= G) {
        return;
    }
#pragma unroll
    for (int b = 0; b < 32; ++b)
        if (cnt[b]) atomicAdd(&counts[32u * w + b], cnt[b]);
}

// Mask bit j = (max(ones, n - ones) >= K), Bitval bit j = Mask && ones > n - ones.
__global__ void k_meta_finalize(const uint32_t* __restrict__ counts, uint32_t Mw, uint64_t n_obs,
                                uint64_t K, uint32_t* __restrict__ mask, uint32_t* __restrict__ bitval) {
    const uint32_t w = blockIdx.x * blockDim.x + threadIdx.x;
    if (w >= Mw) return;
    uint32_t m = 0, v = 0;
    for (int b = 0; b < 32; ++b) {
        uint64_t c1 = counts[32u * w + b];
        uint64_t c0 = n_obs - c1;
        uint64_t agree = c1 > c0 ? c1 : c0;
        if (agree >= K) {
            m |= 1u << b;
            if (c1 > c0) v |= 1u << b;
        }
    }
    mask[w] = m;
    bitval[w] = v;
}

// Derived tables: per position the k, the run shifts and run masks of the
// kept bits; per header-word entry the bit planes of the per-chunk k.
__global__ void k_tables(const uint32_t* __restrict__ mask, const uint32_t* __restrict__ bitval,
                         uint32_t Mw, uint32_t Pc, uint32_t g, uint32_t G, uint32_t* __restrict__ kd,
                         uint32_t* __restrict__ dx, uint32_t* __restrict__ r,
                         uint32_t* __restrict__ planes, Summary* summary) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < Mw) {
        const uint32_t m = mask[i];
        const uint32_t k = (uint32_t)__builtin_popcount(m);
        uint32_t keep = ~m;
        uint32_t src = 0, j = 0;
        uint32_t kdv = k;
        uint32_t dxv[4] = {0, 0, 0, 0};
        while (keep) {
            const uint32_t s = (uint32_t)__builtin_ctz(keep);
            const uint32_t shifted = keep >> s;  // the run starts at bit 0
            const uint32_t len = shifted == 0xFFFFFFFFu ? 32u : (uint32_t)__builtin_ctz(~shifted);
            const uint32_t rm = len == 32 ? 0xFFFFFFFFu : (((1u << len) - 1u) << s);
            const uint32_t d = s - src;
            r[j * Mw + i] = rm;
            if (j < 3)
                kdv |= d << (8 * (j + 1));
            else
                dxv[(j - 3) >> 2] |= d << (8 * ((j - 3) & 3));
            src += len;
            keep &= ~rm;
            ++j;
        }
        for (uint32_t jj = j; jj < (uint32_t)kMaxRuns; ++jj) r[jj * Mw + i] = 0;
        kd[i] = kdv;
        for (int q = 0; q < 4; ++q) dx[q * Mw + i] = dxv[q];
        atomicMax(&summary->max_runs, j);
        atomicAdd(&summary->invariant_bits, (unsigned long long)k);
        if (m != mask[0] || bitval[i] != bitval[0]) atomicAnd(&summary->uniform, 0u);
    }
    const uint32_t Ne = Pc / G;
    if (i < Ne) {
        uint32_t pl[kPlanes];
        for (int q = 0; q < kPlanes; ++q) pl[q] = 0;
        uint32_t kmax = 0;
        for (uint32_t c = 0; c < 32; ++c) {
            const uint32_t cp = (i * G + c) % Pc;
            uint32_t kc = 0;
            for (uint32_t t = 0; t < g; ++t) kc += (uint32_t)__builtin_popcount(mask[cp * g + t]);
            kmax = kc > kmax ? kc : kmax;
            for (int q = 0; q < kPlanes; ++q) pl[q] |= ((kc >> q) & 1u) << c;
        }
        for (int q = 0; q < kPlanes; ++q) planes[(uint64_t)i * kPlanes + q] = pl[q];
        atomicMax(&summary->max_chunk_k, kmax);
    }
}

// ---------------------------------------------------------------------------
// Memory movement helpers (one wave).
// ---------------------------------------------------------------------------

// Copy global words [a, b) of `src` into lds[0 .. b-a).  With `vec`, a and b
// are multiples of 4 and `src` is 16-byte aligned: dwordx4 loads, four in
// flight per lane before the LDS writes.
__device__ __forceinline__ void load_words_to_lds(const uint32_t* __restrict__ src, uint64_t a,
                                                  uint64_t b, uint32_t* lds, bool vec) {
    const uint32_t lane = lane_id();
    if (vec) {
        const uint4* s4 = reinterpret_cast<const uint4*>(src + a);
        uint4* l4 = reinterpret_cast<uint4*>(lds);
        const uint32_t n4 = (uint32_t)((b - a) >> 2);
        uint32_t i = lane;
        for (; i + 3 * kWave < n4; i += 4 * kWave) {
            uint4 v0 = s4[i], v1 = s4[i + kWave], v2 = s4[i + 2 * kWave], v3 = s4[i + 3 * kWave];
            l4[i] = v0;
            l4[i + kWave] = v1;
            l4[i + 2 * kWave] = v2;
            l4[i + 3 * kWave] = v3;
        }
        for (; i < n4; i += kWave) l4[i] = s4[i];
    } else {
        const uint32_t n = (uint32_t)(b - a);
        for (uint32_t i = lane; i < n; i += kWave) lds[i] = src[a + i];
    }
}

// Copy words [w0, w0 + nw) of a raw tensor.
__device__ __forceinline__ void copy_words(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                           uint64_t w0, uint32_t nw, bool vec) {
    const uint32_t lane = lane_id();
    if (vec && (w0 & 3) == 0 && (nw & 3) == 0) {
        const uint4* s4 = reinterpret_cast<const uint4*>(src + w0);
        uint4* d4 = reinterpret_cast<uint4*>(dst + w0);
        const uint32_t n4 = nw >> 2;
        uint32_t i = lane;
        for (; i + 3 * kWave < n4; i += 4 * kWave) {
            uint4 v0 = s4[i], v1 = s4[i + kWave], v2 = s4[i + 2 * kWave], v3 = s4[i + 3 * kWave];
            d4[i] = v0;
            d4[i + kWave] = v1;
            d4[i + 2 * kWave] = v2;
            d4[i + 3 * kWave] = v3;
        }
        for (; i < n4; i += kWave) d4[i] = s4[i];
    } else {
        for (uint32_t i = lane; i < nw; i += kWave) dst[w0 + i] = src[w0 + i];
    }
}

__device__ __forceinline__ void latch_error(uint32_t* err, uint32_t code) {
    if (lane_id() == 0) atomicCAS(err, 0u, code);
}

// ---------------------------------------------------------------------------
// Step 3: decompression of one tile.
// ---------------------------------------------------------------------------

// Rebuild words [w0, w0 + nw) of a tensor.  hdr: the tile's participation
// bits (bit 0 = first chunk of the tile); pay: LDS words holding the tile's
// payload, its first bit at bit `bit0` of pay[0].
template <int RUNS>
__device__ __forceinline__ void decode_steps(const Tables& t, const Geo& geo, const uint32_t* hdr,
                                             const uint32_t* pay, uint32_t bit0, uint64_t w0,
                                             uint32_t nw, uint32_t* __restrict__ out) {
    const uint32_t lane = lane_id();
    const uint32_t Mw = geo.Mw;
    const uint32_t inc = (uint32_t)(kWave % Mw);
    uint32_t pos = (uint32_t)((w0 + lane) % Mw);
    uint32_t carry = bit0;
    const uint32_t steps = (nw + kWave - 1) / kWave;
    for (uint32_t s = 0; s < steps; ++s) {
        const uint32_t lw = s * kWave + lane;  // word within the tile
        const bool valid = lw < nw;
        const uint32_t c = lw >> geo.log2g;    // chunk within the tile
        const uint32_t p = valid ? (hdr[c >> 5] >> (c & 31)) & 1u : 0u;
        const uint32_t kd = t.kd[pos];
        const uint32_t size = valid ? (p ? 32u - (kd & 63u) : 32u) : 0u;
        const uint32_t incl = wave_incl_scan(size);
        const uint32_t off = carry + incl - size;
        carry += lane_value(incl, kWave - 1);
        const uint32_t q = off >> 5, sh = off & 31u;
        const uint32_t f = funnel(pay[q + 1], pay[q], sh);
        uint32_t x = f;
        if (p) x = deposit<RUNS>(t, Mw, pos, kd, t.b[pos], f);
        if (valid) out[w0 + lw] = x;
        pos += inc;
        if (pos >= Mw) pos -= Mw;
    }
}

// Sum over the tile's header words of the removed bits; flags non-zero
// header padding (bits past the last chunk of the tensor).
__device__ __forceinline__ uint32_t tile_removed_bits(const Tables& t, const Geo& geo,
                                                      const uint32_t* hdr, uint64_t hw0,
                                                      uint32_t hw_t, bool* bad_pad) {
    const uint32_t lane = lane_id();
    uint32_t rem = 0;
    bool bad = false;
    for (uint32_t j = lane; j < hw_t; j += kWave) {
        uint32_t h = hdr[j];
        const uint64_t gj = hw0 + j;
        if (gj == geo.hdr_words - 1) {
            const uint32_t valid = (uint32_t)(geo.n_chunks - 32ull * gj);
            if (valid < 32) {
                if (h >> valid) bad = true;
                h &= (1u << valid) - 1u;
            }
        }
        rem += removed_bits(t, geo, gj, h);
    }
    *bad_pad = ballot(bad) != 0;
    return wave_sum(rem);
}

template <int RUNS, bool MULTI>
__global__ __launch_bounds__(256) void k_decode(Tables t, Geo geo, const uint8_t* __restrict__ slots,
                                                uint64_t n_slots, const uint32_t* __restrict__ bitmask,
                                                const int64_t* __restrict__ ids, uint64_t n_out,
                                                uint8_t* __restrict__ dst, uint32_t* err, LookBack lb,
                                                uint32_t lds_words) {
    extern __shared__ uint32_t smem[];
    const uint32_t lane = lane_id();
    uint32_t* lds = smem + (threadIdx.x / kWave) * lds_words;

    uint64_t tile;
    if (MULTI) {
        uint32_t tk = 0;
        if (lane == 0) tk = atomicAdd(lb.ticket, 1u);
        tile = (uint32_t)(uniform(tk) - lb.ticket_base);
    } else {
        tile = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    }
    const uint64_t tpt = MULTI ? geo.tiles_per_tensor : 1;
    if (tile >= n_out * tpt) return;
    const uint64_t oi = MULTI ? tile / tpt : tile;
    const uint64_t local = MULTI ? tile - oi * tpt : 0;

    const int64_t tensor = ids ? (int64_t)uniform64((uint64_t)ids[oi]) : (int64_t)oi;
    if (tensor < 0 || (uint64_t)tensor >= n_slots) {
        latch_error(err, kErrRange);
        return;
    }
    const uint32_t* src = reinterpret_cast<const uint32_t*>(slots + (uint64_t)tensor * geo.L);
    uint32_t* out = reinterpret_cast<uint32_t*>(dst + oi * geo.L);
    const uint64_t w0 = local * geo.tile_words;
    const uint32_t nw = (uint32_t)min((uint64_t)geo.tile_words, geo.n_words - w0);
    const bool vec = geo.aligned16 != 0;
    const bool comp = (uniform(bitmask[(uint64_t)tensor >> 5]) >> ((uint64_t)tensor & 31)) & 1u;
    if (!comp) {
        copy_words(src, out, w0, nw, vec);
        return;
    }

    if (!MULTI) {
        // The whole record: header words, then the payload from word hw on.
        const uint32_t hw = (uint32_t)geo.hdr_words;
        const uint32_t cap = (uint32_t)geo.n_words;  // a record never reaches the slot end
        uint32_t have = geo.spec_words;
        load_words_to_lds(src, 0, have, lds, vec);
        __builtin_amdgcn_wave_barrier();
        bool bad_pad;
        const uint32_t rem = tile_removed_bits(t, geo, lds, 0, hw, &bad_pad);
        const uint64_t R = 32ull * hw + 32ull * geo.n_words - rem;
        const uint64_t words = (R + 31) / 32;
        if (bad_pad || 4 * words >= geo.L) {
            latch_error(err, kErrCorrupt);
            return;
        }
        if (words > have) {
            const uint32_t need = vec ? (uint32_t)((words + 3) & ~3ull) : (uint32_t)words;
            const uint32_t upto = min(need, cap);
            load_words_to_lds(src, have, upto, lds + have, vec);
            have = upto;
        }
        // one zero word past the record keeps the last funnel shift defined
        if (lane == 0) lds[have] = 0;
        __builtin_amdgcn_wave_barrier();
        decode_steps<RUNS>(t, geo, lds, lds + hw, 0, 0, nw, out);
        return;
    }

    // Tile of a long tensor: header slice, look-back, then the payload slice.
    const uint64_t c0 = w0 >> geo.log2g;
    const uint32_t nch = nw >> geo.log2g;
    const uint32_t hw_t = (nch + 31) / 32;
    const uint64_t hw0 = c0 >> 5;
    uint32_t* hdr = lds;
    uint32_t* pay = lds + 64;
    for (uint32_t j = lane; j < hw_t; j += kWave) hdr[j] = src[hw0 + j];
    __builtin_amdgcn_wave_barrier();
    bool bad_pad;
    const uint32_t rem = tile_removed_bits(t, geo, hdr, hw0, hw_t, &bad_pad);
    const uint64_t agg = 32ull * nw - rem;
    const uint64_t S = lookback_exclusive(lb.status, oi * tpt, local, agg, 32ull * geo.hdr_words, lb.epoch);
    const uint64_t E = S + agg;
    const bool last = local == tpt - 1;
    if (bad_pad || E > 8ull * geo.L || (last && 4 * ((E + 31) / 32) >= geo.L)) {
        latch_error(err, kErrCorrupt);
        return;
    }
    uint64_t a = S >> 5, b = (E + 31) >> 5;
    if (vec) {
        a &= ~3ull;
        b = (b + 3) & ~3ull;
    }
    b = min(b, geo.n_words);
    load_words_to_lds(src, a, b, pay, vec);
    if (lane == 0) pay[b - a] = 0;
    __builtin_amdgcn_wave_barrier();
    decode_steps<RUNS>(t, geo, hdr, pay, (uint32_t)(S - 32 * a), w0, nw, out);
}

// ---------------------------------------------------------------------------
// Step 2: compression of one tile.
// ---------------------------------------------------------------------------

// Match test, removal and packing of words [w0, w0 + nw) of tensor x.  The
// participation bits go to hdr (bit 0 = first chunk of the tile), the kept
// bits to pay from bit 0 on; both must be zero on entry.  Returns the payload
// bit count.
template <int RUNS>
__device__ __forceinline__ uint32_t encode_steps(const Tables& t, const Geo& geo,
                                                 const uint32_t* __restrict__ x, uint64_t w0,
                                                 uint32_t nw, uint32_t* hdr, uint32_t* pay) {
    const uint32_t lane = lane_id();
    const uint32_t Mw = geo.Mw;
    const uint32_t inc = (uint32_t)(kWave % Mw);
    const uint32_t g = 1u << geo.log2g;
    const uint64_t gmask = (g >= 64) ? ~0ull : ((1ull << g) - 1);
    uint32_t pos = (uint32_t)((w0 + lane) % Mw);
    uint32_t carry = 0;
    const uint32_t steps = (nw + kWave - 1) / kWave;
    for (uint32_t s = 0; s < steps; ++s) {
        const uint32_t lw = s * kWave + lane;
        const bool valid = lw < nw;
        const uint32_t v = valid ? x[w0 + lw] : 0u;
        const uint32_t m = t.m[pos], b = t.b[pos], kd = t.kd[pos];
        const bool mis = valid && ((v ^ b) & m) != 0;
        bool p;
        if (geo.log2g == 0) {
            p = !mis;
        } else {
            const uint64_t bal = ballot(mis);
            const uint32_t gs = (lane >> geo.log2g) << geo.log2g;
            p = ((bal >> gs) & gmask) == 0;
        }
        const uint32_t c = lw >> geo.log2g;
        if (valid && p && (lw & (g - 1)) == 0) atomicOr(&hdr[c >> 5], 1u << (c & 31));
        const uint32_t f = p ? extract<RUNS>(t, Mw, pos, kd, v) : v;
        const uint32_t size = valid ? (p ? 32u - (kd & 63u) : 32u) : 0u;
        const uint32_t incl = wave_incl_scan(size);
        const uint32_t off = carry + incl - size;
        carry += lane_value(incl, kWave - 1);
        if (size) {
            const uint32_t q = off >> 5, sh = off & 31u;
            atomicOr(&pay[q], f << sh);
            if (sh + size > 32) atomicOr(&pay[q + 1], f >> (32 - sh));
        }
        pos += inc;
        if (pos >= Mw) pos -= Mw;
    }
    return carry;
}

// The r payload bits just before word w0's first payload bit (r in 1..31),
// rebuilt from the source words before w0: returned in bits [0, r).
template <int RUNS>
__device__ uint32_t bits_before_tile(const Tables& t, const Geo& geo, const uint32_t* __restrict__ x,
                                     uint64_t w0, uint32_t r) {
    const uint32_t lane = lane_id();
    const uint32_t g = 1u << geo.log2g;
    const uint64_t gmask = (g >= 64) ? ~0ull : ((1ull << g) - 1);
    uint32_t acc = 0;
    uint64_t after = 0;  // payload bits between the window's end and the tile start
    uint64_t wend = w0;
    while (after < r && wend > 0) {
        const uint64_t wb = wend - kWave;
        const uint64_t w = wb + lane;
        const uint32_t pos = (uint32_t)(w % geo.Mw);
        const uint32_t v = x[w];
        const uint32_t m = t.m[pos], b = t.b[pos], kd = t.kd[pos];
        const bool mis = ((v ^ b) & m) != 0;
        bool p;
        if (geo.log2g == 0) {
            p = !mis;
        } else {
            const uint64_t bal = ballot(mis);
            const uint32_t gs = (lane >> geo.log2g) << geo.log2g;
            p = ((bal >> gs) & gmask) == 0;
        }
        const uint32_t f = p ? extract<RUNS>(t, geo.Mw, pos, kd, v) : v;
        const uint32_t size = p ? 32u - (kd & 63u) : 32u;
        const uint32_t incl = wave_incl_scan(size);
        const uint32_t total = lane_value(incl, kWave - 1);
        const uint64_t end_dist = after + (total - incl);     // bits from field end to tile start
        const uint64_t start_dist = end_dist + size;
        uint32_t contrib = 0;
        if (size && end_dist < r) {
            const int32_t sh = (int32_t)r - (int32_t)start_dist;
            contrib = sh >= 0 ? (f << sh) : (f >> (uint32_t)(-sh));
            contrib &= (1u << r) - 1u;
        }
        acc |= wave_or(contrib);
        after += total;
        wend = wb;
    }
    return acc;
}

template <int RUNS, bool MULTI>
__global__ __launch_bounds__(256) void k_encode(Tables t, Geo geo, const uint8_t* __restrict__ src,
                                                uint64_t n_tensors, uint8_t* __restrict__ slots,
                                                uint32_t* __restrict__ bitmask, uint64_t* __restrict__ stored,
                                                LookBack lb, uint32_t lds_words) {
    extern __shared__ uint32_t smem[];
    const uint32_t lane = lane_id();
    uint32_t* lds = smem + (threadIdx.x / kWave) * lds_words;

    uint64_t tile;
    if (MULTI) {
        uint32_t tk = 0;
        if (lane == 0) tk = atomicAdd(lb.ticket, 1u);
        tile = (uint32_t)(uniform(tk) - lb.ticket_base);
    } else {
        tile = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    }
    const uint64_t tpt = MULTI ? geo.tiles_per_tensor : 1;
    if (tile >= n_tensors * tpt) return;
    const uint64_t ti = MULTI ? tile / tpt : tile;
    const uint64_t local = MULTI ? tile - ti * tpt : 0;
    const uint32_t* x = reinterpret_cast<const uint32_t*>(src + ti * geo.L);
    uint32_t* slot = reinterpret_cast<uint32_t*>(slots + ti * geo.L);
    const uint64_t w0 = local * geo.tile_words;
    const uint32_t nw = (uint32_t)min((uint64_t)geo.tile_words, geo.n_words - w0);
    const bool vec = geo.aligned16 != 0;

    uint32_t* hdr = lds;
    uint32_t* pay = lds + 64;
    for (uint32_t i = lane; i < 64 + nw + 2; i += kWave) lds[i] = 0;
    __builtin_amdgcn_wave_barrier();
    const uint32_t agg = encode_steps<RUNS>(t, geo, x, w0, nw, hdr, pay);
    __builtin_amdgcn_wave_barrier();

    if (!MULTI) {
        const uint32_t hw = (uint32_t)geo.hdr_words;
        const uint64_t R = 32ull * hw + agg;
        const uint64_t words = (R + 31) / 32;
        const bool comp = 4 * words < geo.L;
        if (comp) {
            for (uint32_t i = lane; i < hw; i += kWave) slot[i] = hdr[i];
            for (uint32_t i = lane; i < words - hw; i += kWave) slot[hw + i] = pay[i];
        } else {
            copy_words(x, slot, 0, (uint32_t)geo.n_words, vec);
        }
        if (lane == 0) {
            const uint32_t bit = 1u << (ti & 31);
            if (comp)
                atomicOr(&bitmask[ti >> 5], bit);
            else
                atomicAnd(&bitmask[ti >> 5], ~bit);
            if (stored) stored[ti] = comp ? 4 * words : geo.L;
        }
        return;
    }

    const uint64_t S = lookback_exclusive(lb.status, ti * tpt, local, agg, 32ull * geo.hdr_words, lb.epoch);
    const uint64_t E = S + agg;
    const bool last = local == tpt - 1;
    // header words of this tile (always inside the slot)
    const uint64_t hw0 = (w0 >> geo.log2g) >> 5;
    const uint32_t hw_t = ((nw >> geo.log2g) + 31) / 32;
    for (uint32_t j = lane; j < hw_t; j += kWave) slot[hw0 + j] = hdr[j];
    // Words whose last bit lies in [S, E) belong to this tile; the final
    // partial word (zero padded) belongs to the last tile.
    const uint64_t q0 = S >> 5;
    uint64_t q1 = E >> 5;  // exclusive
    if (last && (E & 31)) q1 += 1;
    q1 = min(q1, geo.n_words);  // an incompressible tensor is rewritten raw later
    const uint32_t r = (uint32_t)(S & 31);
    uint32_t prev = 0;
    if (r && q0 < q1) prev = bits_before_tile<RUNS>(t, geo, x, w0, r);
    for (uint64_t q = q0 + lane; q < q1; q += kWave) {
        const int64_t u = (int64_t)(32 * q) - (int64_t)S;
        uint32_t val;
        if (u < 0) {
            val = (pay[0] << r) | prev;
        } else {
            const uint32_t uq = (uint32_t)(u >> 5);
            val = funnel(pay[uq + 1], pay[uq], (uint32_t)(u & 31));
        }
        slot[q] = val;
    }
    if (last && lane == 0) lb.totals[ti] = E;
}

// After the tiles of long tensors: bitmask bit, stored bytes, and the raw
// copy of a tensor whose record is not shorter than its slot.
__global__ __launch_bounds__(256) void k_encode_finalize(Geo geo, const uint8_t* __restrict__ src,
                                                         uint8_t* __restrict__ slots,
                                                         uint32_t* __restrict__ bitmask,
                                                         uint64_t* __restrict__ stored,
                                                         const uint64_t* __restrict__ totals,
                                                         uint32_t blocks_per_tensor) {
    const uint64_t ti = blockIdx.x / blocks_per_tensor;
    const uint32_t bi = blockIdx.x % blocks_per_tensor;
    const uint64_t E = totals[ti];
    const uint64_t words = (E + 31) / 32;
    const bool comp = 4 * words < geo.L;
    if (bi == 0 && threadIdx.x == 0) {
        const uint32_t bit = 1u << (ti & 31);
        if (comp)
            atomicOr(&bitmask[ti >> 5], bit);
        else
            atomicAnd(&bitmask[ti >> 5], ~bit);
        if (stored) stored[ti] = comp ? 4 * words : geo.L;
    }
    if (comp) return;
    const uint32_t* x = reinterpret_cast<const uint32_t*>(src + ti * geo.L);
    uint32_t* slot = reinterpret_cast<uint32_t*>(slots + ti * geo.L);
    for (uint64_t i = (uint64_t)bi * blockDim.x + threadIdx.x; i < geo.n_words;
         i += (uint64_t)blocks_per_tensor * blockDim.x)
        slot[i] = x[i];
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_meta_hist(const uint32_t* sample, uint64_t n_words, uint32_t Mw, uint32_t* counts,
                            hipStream_t s) {
    const uint64_t n_obs = n_words / Mw;
    uint64_t reps = (256ull * 1024 + Mw - 1) / Mw;
    if (reps > n_obs) reps = n_obs;
    if (reps == 0) reps = 1;
    const uint64_t G = reps * Mw;
    const uint64_t blocks = (G + 255) / 256;
    hipLaunchKernelGGL(k_meta_hist, dim3((uint32_t)blocks), dim3(256), 0, s, sample, n_words, Mw, G, counts);
    return hipGetLastError();
}

hipError_t launch_meta_finalize(const uint32_t* counts, uint32_t Mw, uint64_t n_obs, uint64_t K,
                                uint32_t* mask, uint32_t* bitval, hipStream_t s) {
    hipLaunchKernelGGL(k_meta_finalize, dim3((Mw + 255) / 256), dim3(256), 0, s, counts, Mw, n_obs, K,
                       mask, bitval);
    return hipGetLastError();
}

hipError_t launch_tables(const uint32_t* mask, const uint32_t* bitval, uint32_t Mw, uint32_t Pc,
                         uint32_t g, uint32_t G, uint32_t* kd, uint32_t* dx, uint32_t* r,
                         uint32_t* planes, Summary* summary, hipStream_t s) {
    const uint32_t n = Mw > Pc / G ? Mw : Pc / G;
    hipLaunchKernelGGL(k_tables, dim3((n + 255) / 256), dim3(256), 0, s, mask, bitval, Mw, Pc, g, G, kd,
                       dx, r, planes, summary);
    return hipGetLastError();
}

static uint32_t runs_bucket(uint32_t runs) {
    if (runs <= 4) return runs;
    if (runs <= 8) return 8;
    return 16;
}

template <bool MULTI>
static hipError_t launch_decode_t(const Tables& t, const Geo& geo, uint32_t runs, const void* slots,
                                  uint64_t n_slots, const uint32_t* bitmask, const int64_t* ids,
                                  uint64_t n_out, void* dst, uint32_t* err, const LookBack& lb,
                                  uint32_t lds_words, hipStream_t s) {
    const uint64_t tiles = n_out * geo.tiles_per_tensor;
    const dim3 grid((uint32_t)((tiles + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(kWave * kWavesPerBlock);
    const size_t shm = (size_t)lds_words * 4 * kWavesPerBlock;
    const uint8_t* sl = static_cast<const uint8_t*>(slots);
    uint8_t* d = static_cast<uint8_t*>(dst);
#define IBP_DEC(R)                                                                                  \
    hipLaunchKernelGGL((k_decode<R, MULTI>), grid, block, shm, s, t, geo, sl, n_slots, bitmask, ids, \
                       n_out, d, err, lb, lds_words)
    switch (runs_bucket(runs)) {
        case 0: IBP_DEC(0); break;
        case 1: IBP_DEC(1); break;
        case 2: IBP_DEC(2); break;
        case 3: IBP_DEC(3); break;
        case 4: IBP_DEC(4); break;
        case 8: IBP_DEC(8); break;
        default: IBP_DEC(16); break;
    }
#undef IBP_DEC
    return hipGetLastError();
}

hipError_t launch_decode(const Tables& t, const Geo& geo, uint32_t runs, const void* slots,
                         uint64_t n_slots, const uint32_t* bitmask, const int64_t* ids,
                         uint64_t n_out, void* dst, uint32_t* err, const LookBack* lb, hipStream_t s) {
    if (n_out == 0) return hipSuccess;
    if (geo.tiles_per_tensor == 1) {
        const uint32_t lds_words = (uint32_t)geo.n_words + 8;
        return launch_decode_t<false>(t, geo, runs, slots, n_slots, bitmask, ids, n_out, dst, err,
                                      LookBack{}, lds_words, s);
    }
    const uint32_t lds_words = 64 + geo.tile_words + 8;
    return launch_decode_t<true>(t, geo, runs, slots, n_slots, bitmask, ids, n_out, dst, err, *lb,
                                 lds_words, s);
}

template <bool MULTI>
static hipError_t launch_encode_t(const Tables& t, const Geo& geo, uint32_t runs, const void* src,
                                  uint64_t n_tensors, void* slots, uint32_t* bitmask, uint64_t* stored,
                                  const LookBack& lb, uint32_t lds_words, hipStream_t s) {
    const uint64_t tiles = n_tensors * geo.tiles_per_tensor;
    const dim3 grid((uint32_t)((tiles + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(kWave * kWavesPerBlock);
    const size_t shm = (size_t)lds_words * 4 * kWavesPerBlock;
    const uint8_t* sr = static_cast<const uint8_t*>(src);
    uint8_t* sl = static_cast<uint8_t*>(slots);
#define IBP_ENC(R)                                                                                \
    hipLaunchKernelGGL((k_encode<R, MULTI>), grid, block, shm, s, t, geo, sr, n_tensors, sl, bitmask, \
                       stored, lb, lds_words)
    switch (runs_bucket(runs)) {
        case 0: IBP_ENC(0); break;
        case 1: IBP_ENC(1); break;
        case 2: IBP_ENC(2); break;
        case 3: IBP_ENC(3); break;
        case 4: IBP_ENC(4); break;
        case 8: IBP_ENC(8); break;
        default: IBP_ENC(16); break;
    }
#undef IBP_ENC
    return hipGetLastError();
}

hipError_t launch_encode(const Tables& t, const Geo& geo, uint32_t runs, const void* src,
                         uint64_t n_tensors, void* slots, uint32_t* bitmask, uint64_t* stored,
                         const LookBack* lb, hipStream_t s) {
    if (n_tensors == 0) return hipSuccess;
    const uint32_t lds_words = 64 + geo.tile_words + 8;
    if (geo.tiles_per_tensor == 1)
        return launch_encode_t<false>(t, geo, runs, src, n_tensors, slots, bitmask, stored, LookBack{},
                                      lds_words, s);
    hipError_t e = launch_encode_t<true>(t, geo, runs, src, n_tensors, slots, bitmask, stored, *lb,
                                         lds_words, s);
    if (e != hipSuccess) return e;
    uint64_t per = (geo.n_words + 256ull * 64 - 1) / (256ull * 64);  // ~64 words per thread
    if (per > 1024) per = 1024;
    const uint32_t bpt = (uint32_t)(per ? per : 1);
    hipLaunchKernelGGL(k_encode_finalize, dim3((uint32_t)(n_tensors * bpt)), dim3(256), 0, s, geo,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(slots), bitmask, stored,
                       lb->totals, bpt);
    return hipGetLastError();
}

}  // namespace ibp

namespace ibp {

__global__ void k_fill_u32(uint32_t* __restrict__ p, uint64_t n, uint32_t v) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, uint64_t n, uint32_t v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_fill_u32, dim3((uint32_t)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace ibp
