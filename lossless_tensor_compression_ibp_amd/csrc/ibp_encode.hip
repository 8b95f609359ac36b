// ibp_encode.hip -- step 2 of Invariant Bit Packing on gfx950: compression.
//
// Method: FR summary ("Résumé Technique : Réduire le goulot d'étranglement de
// la mémoire GPU par la compression sans perte pour le ML") and KO summary
// ("Reducing the GPU Memory Bottleneck with Lossless Compression for ML --
// Extended"), section "Algorithme central" / "핵심 알고리즘", step 2: each
// chunk is tested against Bitval at the masked positions; a matching chunk
// loses those bits and its other bits close up; every chunk carries a
// participation bit.  Section "Intégration au système": records go into
// fixed-size slots and a GPU bitmask says which slots hold a record.
//
// One wave64 encodes one tile (all of a tensor of at most 2048 words, or a
// 1024-word tile of a longer one); tiles of one tensor find their start bit
// by decoupled look-back.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ibp_device.hpp"
#include "ibp_internal.hpp"

namespace ibp {

static uint32_t runs_bucket(uint32_t runs) {
    if (runs <= 4) return runs;
    if (runs <= 8) return 8;
    return 16;
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
