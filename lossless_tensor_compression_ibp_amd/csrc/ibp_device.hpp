// ibp_device.hpp -- wave64 building blocks for the IBP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ibp_internal.hpp"

namespace ibp {

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    uint32_t lo = uniform((uint32_t)v);
    uint32_t hi = uniform((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t lane_value(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` below this lane (v_mbcnt_lo/hi).
__device__ __forceinline__ uint32_t bits_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive wave64 prefix sum with DPP: row_shr 1/2/4/8 inside 16-lane rows,
// then row_bcast:15 and row_bcast:31 carry row totals upward.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
    return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
    return lane_value(wave_incl_scan(x), kWave - 1);
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t x) {
    for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
    for (int o = kWave / 2; o > 0; o >>= 1) x |= (uint32_t)__shfl_xor((int)x, o);
    return x;
}

// ((hi:lo) >> sh) & 0xffffffff, sh in [0, 31]
__device__ __forceinline__ uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t sh) {
    return __builtin_amdgcn_alignbit(hi, lo, sh);
}

// ---------------------------------------------------------------------------
// Removal and reinsertion of masked bits with a run table.  The kept bits
// (~Mask) of a word form at most 16 runs; run j covers output bits R_j and is
// fed by the field bits starting d_j places lower.  Reinsertion (a PDEP on
// ~Mask) is OR_j ((f << d_j) & R_j); removal (a PEXT on ~Mask) is
// OR_j ((x & R_j) >> d_j).
// ---------------------------------------------------------------------------
template <int RUNS>
__device__ __forceinline__ uint32_t run_shift(const Tables& t, uint32_t Mw, uint32_t pos,
                                              uint32_t kd, int j) {
    if (j < 3) return kd >> (8 * (j + 1));
    return t.dx[(uint32_t)((j - 3) >> 2) * Mw + pos] >> (8 * ((j - 3) & 3));
}

template <int RUNS>
__device__ __forceinline__ uint32_t deposit(const Tables& t, uint32_t Mw, uint32_t pos, uint32_t kd,
                                            uint32_t bitval, uint32_t f) {
    uint32_t x = bitval;
#pragma unroll
    for (int j = 0; j < RUNS; ++j) {
        uint32_t d = run_shift<RUNS>(t, Mw, pos, kd, j) & 31u;
        uint32_t r = t.r[(uint32_t)j * Mw + pos];
        x |= (f << d) & r;
    }
    return x;
}

template <int RUNS>
__device__ __forceinline__ uint32_t extract(const Tables& t, uint32_t Mw, uint32_t pos, uint32_t kd,
                                            uint32_t x) {
    uint32_t f = 0;
#pragma unroll
    for (int j = 0; j < RUNS; ++j) {
        uint32_t d = run_shift<RUNS>(t, Mw, pos, kd, j) & 31u;
        uint32_t r = t.r[(uint32_t)j * Mw + pos];
        f |= (x & r) >> d;
    }
    return f;
}

// Bits of the header word `hword` (global header word index j) that stand for
// removed bits: sum over set participation bits of that chunk's k, from the
// bit planes of entry ((32 j) mod Pc) / G.
__device__ __forceinline__ uint32_t removed_bits(const Tables& t, const Geo& g, uint64_t j,
                                                 uint32_t hword) {
    uint32_t e = (uint32_t)(((32ull * j) % g.Pc) / g.G);
    const uint32_t* pl = t.planes + (uint64_t)e * kPlanes;
    uint32_t s = 0;
    for (uint32_t q = 0; q < g.np; ++q) s += (uint32_t)__builtin_popcount(hword & pl[q]) << q;
    return s;
}

// ---------------------------------------------------------------------------
// Decoupled look-back across the tiles of one tensor.
// ---------------------------------------------------------------------------
constexpr uint32_t kFlagAgg = 1, kFlagIncl = 2;
constexpr uint64_t kValMask = (1ull << 42) - 1;

__device__ __forceinline__ unsigned long long pack_status(uint32_t flag, uint32_t epoch, uint64_t v) {
    return ((unsigned long long)flag << 62) | ((unsigned long long)(epoch & 0xFFFFFu) << 42) |
           (v & kValMask);
}

__device__ __forceinline__ void status_store(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long status_load(unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tile `local` of a tensor whose tiles use status[first .. first+n); returns
// the sum of `base` and the aggregates of every earlier tile, and publishes
// this tile's inclusive value.  Waits only on earlier tiles, which took their
// tickets before this one and are therefore resident or finished.
__device__ uint64_t lookback_exclusive(unsigned long long* status, uint64_t first, uint64_t local,
                                       uint64_t agg, uint64_t base, uint32_t epoch) {
    const uint32_t lane = lane_id();
    unsigned long long* mine = status + first + local;
    if (local == 0) {
        if (lane == 0) status_store(mine, pack_status(kFlagIncl, epoch, base + agg));
        return base;
    }
    if (lane == 0) status_store(mine, pack_status(kFlagAgg, epoch, agg));
    uint64_t excl = 0;
    int64_t j = (int64_t)local - 1;  // newest predecessor not yet summed
    while (true) {
        const bool inwin = (int64_t)lane <= j;
        uint64_t v = 0;
        uint32_t f = 0;
        if (inwin) {
            unsigned long long* p = status + first + (uint64_t)(j - (int64_t)lane);
            while (true) {
                unsigned long long s = status_load(p);
                uint32_t ep = (uint32_t)(s >> 42) & 0xFFFFFu;
                f = (uint32_t)(s >> 62);
                if (f != 0 && ep == (epoch & 0xFFFFFu)) {
                    v = s & kValMask;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        const uint64_t incl = ballot(inwin && f == kFlagIncl);
        if (incl) {
            const uint32_t stop = (uint32_t)__builtin_ctzll(incl);
            excl += wave_sum64(lane <= stop ? v : 0);
            break;
        }
        excl += wave_sum64(v);
        j -= kWave;
    }
    if (lane == 0) status_store(mine, pack_status(kFlagIncl, epoch, excl + agg));
    return excl;
}

}  // namespace ibp
