// ibp_device.hpp -- wave64 building blocks for the IBP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ibp_internal.hpp"

namespace ibp {

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, each index a
// compile-time constant from the start, so a register array indexed by it is
// never turned into one vector that every partial update copies (which a
// loop that is unrolled only later can lead to).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(static_cast<F&&>(f));
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
// Table accessors.  The per-position tables (structure of arrays, stride Mw)
// are read either from arrays (staged in LDS or left in global memory) or,
// when every position holds the same Mask/Bitval word, from wave-uniform
// registers.
// ---------------------------------------------------------------------------
struct TabArrays {
    const uint32_t* b;
    const uint32_t* kd;
    const uint32_t* dx;
    const uint32_t* r;
    uint32_t Mw;
    __device__ __forceinline__ uint32_t kdw(uint32_t pos) const { return kd[pos]; }
    __device__ __forceinline__ uint32_t bw(uint32_t pos) const { return b[pos]; }
    __device__ __forceinline__ uint32_t rw(int j, uint32_t pos) const { return r[(uint32_t)j * Mw + pos]; }
    __device__ __forceinline__ uint32_t dw(int j, uint32_t pos, uint32_t kdv) const {
        if (j < 3) return kdv >> (8 * (j + 1));
        return dx[(uint32_t)((j - 3) >> 2) * Mw + pos] >> (8 * ((j - 3) & 3));
    }
    // four consecutive positions starting at a multiple of 4 (Mw % 4 == 0)
    __device__ __forceinline__ u32x4 kdw4(uint32_t pos) const { return *reinterpret_cast<const u32x4*>(kd + pos); }
    __device__ __forceinline__ u32x4 bw4(uint32_t pos) const { return *reinterpret_cast<const u32x4*>(b + pos); }
    __device__ __forceinline__ u32x4 rw4(int j, uint32_t pos) const {
        return *reinterpret_cast<const u32x4*>(r + (uint32_t)j * Mw + pos);
    }
    __device__ __forceinline__ u32x4 dxw4(int q, uint32_t pos) const {
        return *reinterpret_cast<const u32x4*>(dx + (uint32_t)q * Mw + pos);
    }
    // two consecutive positions starting at an even one (Mw % 4 == 0)
    __device__ __forceinline__ u32x2 kdw2(uint32_t pos) const { return *reinterpret_cast<const u32x2*>(kd + pos); }
    __device__ __forceinline__ u32x2 bw2(uint32_t pos) const { return *reinterpret_cast<const u32x2*>(b + pos); }
    __device__ __forceinline__ u32x2 rw2(int j, uint32_t pos) const {
        return *reinterpret_cast<const u32x2*>(r + (uint32_t)j * Mw + pos);
    }
};

template <int RUNS>
struct TabUniform {
    uint32_t kdv, bv;
    uint32_t r[RUNS > 0 ? RUNS : 1];
    uint32_t d[RUNS > 0 ? RUNS : 1];
    __device__ __forceinline__ uint32_t kdw(uint32_t) const { return kdv; }
    __device__ __forceinline__ uint32_t bw(uint32_t) const { return bv; }
    __device__ __forceinline__ uint32_t rw(int j, uint32_t) const { return r[j]; }
    __device__ __forceinline__ uint32_t dw(int j, uint32_t, uint32_t) const { return d[j]; }
};

template <class Tab>
struct IsUniformTab { static constexpr bool value = false; };
template <int R>
struct IsUniformTab<TabUniform<R>> { static constexpr bool value = true; };

// Position-0 entries of the global tables, moved to scalar registers.
template <int RUNS>
__device__ __forceinline__ TabUniform<RUNS> load_uniform(const Tables& t, uint32_t Mw) {
    TabUniform<RUNS> u;
    u.kdv = uniform(t.kd[0]);
    u.bv = uniform(t.b[0]);
#pragma unroll
    for (int j = 0; j < RUNS; ++j) {
        u.r[j] = uniform(t.r[(uint32_t)j * Mw]);
        u.d[j] = j < 3 ? (u.kdv >> (8 * (j + 1))) & 31u
                       : (uniform(t.dx[(uint32_t)((j - 3) >> 2) * Mw]) >> (8 * ((j - 3) & 3))) & 31u;
    }
    return u;
}

template <int RUNS, class Tab>
__device__ __forceinline__ uint32_t deposit_t(const Tab& tab, uint32_t pos, uint32_t kdv, uint32_t f) {
    uint32_t x = tab.bw(pos);
#pragma unroll
    for (int j = 0; j < RUNS; ++j) x |= (f << (tab.dw(j, pos, kdv) & 31u)) & tab.rw(j, pos);
    return x;
}

template <int RUNS, class Tab>
__device__ __forceinline__ uint32_t extract_t(const Tab& tab, uint32_t pos, uint32_t kdv, uint32_t x) {
    uint32_t f = 0;
#pragma unroll
    for (int j = 0; j < RUNS; ++j) f |= (x & tab.rw(j, pos)) >> (tab.dw(j, pos, kdv) & 31u);
    return f;
}

// Words of LDS the per-position arrays of RUNS runs take (b, kd, dx rows, r rows).
__host__ __device__ constexpr uint32_t dx_rows(int runs) { return runs > 3 ? (uint32_t)(runs - 3 + 3) / 4 : 0u; }
__host__ __device__ constexpr uint32_t tab_rows(int runs) { return 2u + dx_rows(runs) + (uint32_t)runs; }

// Word `e` of rows [row0, row0 + nrows) of the table image m, b, kd, dx rows
// (DXR of them), r rows, each Mw words, in device memory.  The dx and r rows
// are each one array, so a word's source takes compares and selects, no
// division (e differs across lanes).
template <uint32_t DXR>
__device__ __forceinline__ const uint32_t* table_image_word(const Tables& t, uint32_t row0, uint32_t Mw,
                                                            uint32_t e) {
    const uint32_t a = row0 * Mw + e;  // word of the whole image
    const uint32_t* p = a < Mw ? t.m + a : t.b + (a - Mw);
    p = a >= 2 * Mw ? t.kd + (a - 2 * Mw) : p;
    if (DXR > 0) p = a >= 3 * Mw ? t.dx + (a - 3 * Mw) : p;
    p = a >= (3 + DXR) * Mw ? t.r + (a - (3 + DXR) * Mw) : p;
    return p;
}

// Whole workgroup: rows [row0, row0 + nrows) of the table image into lds,
// then n_extra words of `extra` right after them.  A thread issues all loads
// of a round (four 16-byte vectors when Mw is a multiple of 4, else eight
// words) before its LDS writes, and the first two extra words per thread are
// loaded ahead of the table rounds, so staging costs one memory latency per
// round rather than one per element.
template <uint32_t DXR>
__device__ __forceinline__ void stage_table_image(const Tables& t, uint32_t row0, uint32_t nrows, uint32_t Mw,
                                                  const uint32_t* __restrict__ extra, uint32_t n_extra,
                                                  uint32_t* lds) {
    const uint32_t tid = threadIdx.x, nt = blockDim.x;
    const uint32_t tab = nrows * Mw;
    uint32_t ev[2] = {0u, 0u};
#pragma unroll
    for (uint32_t u = 0; u < 2; ++u) {
        const uint32_t e = u * nt + tid;
        if (e < n_extra) ev[u] = extra[e];
    }
    if ((Mw & 3u) == 0) {
        const uint32_t nv = tab >> 2;
        for (uint32_t base = 0; base < nv; base += 4 * nt) {
            u32x4 v[4];
#pragma unroll
            for (uint32_t u = 0; u < 4; ++u) {
                // past the end: a load of the last vector again (no branch
                // around the load, so all four stay in flight together)
                const uint32_t e = min(base + u * nt + tid, nv - 1);
                v[u] = *reinterpret_cast<const u32x4*>(table_image_word<DXR>(t, row0, Mw, 4 * e));
            }
#pragma unroll
            for (uint32_t u = 0; u < 4; ++u) {
                const uint32_t e = base + u * nt + tid;
                if (e < nv) reinterpret_cast<u32x4*>(lds)[e] = v[u];
            }
        }
    } else {
        for (uint32_t base = 0; base < tab; base += 8 * nt) {
            uint32_t v[8];
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u) {
                const uint32_t e = min(base + u * nt + tid, tab - 1);
                v[u] = *table_image_word<DXR>(t, row0, Mw, e);
            }
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u) {
                const uint32_t e = base + u * nt + tid;
                if (e < tab) lds[e] = v[u];
            }
        }
    }
#pragma unroll
    for (uint32_t u = 0; u < 2; ++u) {
        const uint32_t e = u * nt + tid;
        if (e < n_extra) lds[tab + e] = ev[u];
    }
    for (uint32_t e = 2 * nt + tid; e < n_extra; e += nt) lds[tab + e] = extra[e];
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

// Copy global words [a, b) of `src` into lds[0 .. b-a) with non-temporal
// loads and no over-read: dwordx4 for whole 16-byte groups (a is a multiple
// of 4, src 16-byte aligned), single dwords for the tail.  Used for the part
// of a record read after its header, where bytes past the record would only
// cost link or HBM bandwidth.
__device__ __forceinline__ void load_exact_to_lds(const uint32_t* __restrict__ src, uint64_t a, uint64_t b,
                                                  uint32_t* lds) {
    const uint32_t lane = lane_id();
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src + a);
    u32x4* l4 = reinterpret_cast<u32x4*>(lds);
    const uint32_t n = (uint32_t)(b - a);
    const uint32_t n4 = n >> 2;
    uint32_t i = lane;
    for (; i + 3 * kWave < n4; i += 4 * kWave) {
        const u32x4 v0 = __builtin_nontemporal_load(s4 + i), v1 = __builtin_nontemporal_load(s4 + i + kWave);
        const u32x4 v2 = __builtin_nontemporal_load(s4 + i + 2 * kWave);
        const u32x4 v3 = __builtin_nontemporal_load(s4 + i + 3 * kWave);
        l4[i] = v0;
        l4[i + kWave] = v1;
        l4[i + 2 * kWave] = v2;
        l4[i + 3 * kWave] = v3;
    }
    for (; i < n4; i += kWave) l4[i] = __builtin_nontemporal_load(s4 + i);
    if (lane < (n & 3u)) lds[4 * n4 + lane] = __builtin_nontemporal_load(src + a + 4 * n4 + lane);
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

// Removed bits of header word `hword` (global header word index j): the sum
// over its set participation bits of that chunk's k, from the bit planes of
// entry ((32 j) mod Pc) / G (with one chunk per period, every chunk's k).
__device__ __forceinline__ uint32_t removed_bits_pl(const uint32_t* planes, const Geo& g, uint64_t j,
                                                    uint32_t hword) {
    if (g.Pc == 1) return (uint32_t)__builtin_popcount(hword) * g.k1;
    const uint32_t e = (uint32_t)(((32ull * j) % g.Pc) / g.G);
    const uint32_t* pl = planes + e * (uint32_t)kPlanes;
    uint32_t s = 0;
    for (uint32_t q = 0; q < g.np; ++q) s += (uint32_t)__builtin_popcount(hword & pl[q]) << q;
    return s;
}

// Sum over the tile's header words [hw0, hw0 + hw_t) of the removed bits;
// flags non-zero header padding (bits past the tensor's last chunk).
__device__ __forceinline__ uint32_t header_removed_bits(const uint32_t* planes, const Geo& geo,
                                                        const uint32_t* hdr, uint64_t hw0, uint32_t hw_t,
                                                        bool* bad_pad) {
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
        rem += removed_bits_pl(planes, geo, gj, h);
    }
    *bad_pad = ballot(bad) != 0;
    return wave_sum(rem);
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
// tickets before this one and are therefore resident or finished.  A wait
// that outlasts kLookbackPolls polls latches kErrStall in err and returns
// (and publishes) kLookbackPoison, so every wave still exits.
__device__ uint64_t lookback_exclusive(unsigned long long* status, uint64_t first, uint64_t local,
                                       uint64_t agg, uint64_t base, uint32_t epoch, uint32_t* err) {
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
        bool gave_up = false;
        if (inwin) {
            unsigned long long* p = status + first + (uint64_t)(j - (int64_t)lane);
            for (uint32_t polls = 0;; ++polls) {
                unsigned long long s = status_load(p);
                uint32_t ep = (uint32_t)(s >> 42) & 0xFFFFFu;
                f = (uint32_t)(s >> 62);
                if (f != 0 && ep == (epoch & 0xFFFFFu)) {
                    v = s & kValMask;
                    break;
                }
                if (polls >= kLookbackPolls) {
                    gave_up = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (ballot(gave_up)) {
            latch_error(err, kErrStall);
            if (lane == 0) status_store(mine, pack_status(kFlagIncl, epoch, kLookbackPoison));
            return kLookbackPoison;
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
