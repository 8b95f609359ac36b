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
// 1024-word tile of a longer one).  The tiles of a longer tensor find their
// start bits by decoupled look-back when the source is in pinned host memory;
// a source in HBM is read twice instead (a pass summing each group of tiles'
// payload bits, a scan per tensor), and one wave encodes a group of tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
        tile = uniform(tk);
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

    const uint64_t S = lookback_exclusive(lb.status, ti * tpt, local, agg, 32ull * geo.hdr_words, lb.epoch, lb.err);
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

// Tables one encode step reads: the Mask row and the per-position arrays (in
// LDS or global memory), or for uniform metadata the position-0 entries in
// registers.
template <int RUNS, bool UNI>
struct EncTabs {
    static constexpr bool kRegs = false;
    const uint32_t* mrow;
    TabArrays ta;
    TabUniform<RUNS> tu;
    uint32_t mu;
};

// The same entries for one lane's NW consecutive positions (Mw a multiple of
// 4, at most three runs), loaded once into registers.
template <int RUNS, int NW>
struct EncRegs {
    static_assert(RUNS <= 3, "run shifts past the third live in the dx rows");
    static constexpr bool kRegs = true;
    using V = std::conditional_t<NW == 4, u32x4, u32x2>;
    V m, b, kd;
    V r[RUNS > 0 ? RUNS : 1];
    TabUniform<RUNS> tu;  // unused
    uint32_t mu = 0;      // unused
    __device__ __forceinline__ void load(const Tables& t, uint32_t Mw, uint32_t pos0) {
        m = *reinterpret_cast<const V*>(t.m + pos0);
        b = *reinterpret_cast<const V*>(t.b + pos0);
        kd = *reinterpret_cast<const V*>(t.kd + pos0);
#pragma unroll
        for (int j = 0; j < RUNS; ++j) r[j] = *reinterpret_cast<const V*>(t.r + (uint32_t)j * Mw + pos0);
    }
};

template <int RUNS, bool UNI>
__device__ __forceinline__ EncTabs<RUNS, UNI> enc_tabs_global(const Tables& t, uint32_t Mw) {
    EncTabs<RUNS, UNI> e{};
    e.mrow = t.m;
    e.ta = TabArrays{t.b, t.kd, t.dx, t.r, Mw};
    if constexpr (UNI) {
        e.tu = load_uniform<RUNS>(t, Mw);
        e.mu = uniform(t.m[0]);
    }
    return e;
}

// NW consecutive table words from p (p 4 * NW-byte aligned).
template <int NW>
__device__ __forceinline__ void load_vec(const uint32_t* p, uint32_t (&v)[NW]) {
    if constexpr (NW == 4) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = w[j];
    } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(p);
        v[0] = w[0];
        v[1] = w[1];
    }
}

// One lane's share of an encode step: the match test, participation and
// removal of its NW (4, or 2 for tensors of at most 128 words) consecutive
// words x, at positions pos0.. of the period (all live or none).  With HDR the
// lane's participation bits are OR-ed into hdr from chunk c0, its first
// word's; each word's field goes to f and its width to size; returns the
// widths' sum.  Every lane of the wave calls it (chunks longer than a lane's
// words take a ballot).  With two words per lane and W = 32 the step's first
// chunk must start a header word (c0 = that chunk + 2 * lane).
template <int NW, int RUNS, bool UNI, bool MW4, bool HDR, class ET = EncTabs<RUNS, UNI>>
__device__ __forceinline__ uint32_t encode_lane(const ET& et, uint32_t Mw, uint32_t lg, bool live,
                                                uint32_t pos0, const uint32_t (&x)[NW], uint32_t* hdr, uint32_t c0,
                                                uint32_t (&f)[NW], uint32_t (&size)[NW]) {
    static_assert(NW == 2 || NW == 4, "two or four words per lane");
    constexpr bool REGS = ET::kRegs;
    const uint32_t lane = lane_id();
    const uint32_t g = 1u << lg;
    const TabUniform<RUNS>& tu = et.tu;
    const uint32_t mu = et.mu;
    uint32_t m[NW], bv[NW], kd[NW], pos[NW];
    if constexpr (REGS) {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            pos[j] = pos0 + j;
            m[j] = et.m[j];
            bv[j] = et.b[j];
            kd[j] = et.kd[j];
        }
    } else if constexpr (UNI) {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            pos[j] = 0;
            m[j] = mu;
            bv[j] = tu.bw(0);
            kd[j] = tu.kdw(0);
        }
    } else if constexpr (MW4) {
        load_vec<NW>(et.mrow + pos0, m);
        load_vec<NW>(et.ta.b + pos0, bv);
        load_vec<NW>(et.ta.kd + pos0, kd);
#pragma unroll
        for (int j = 0; j < NW; ++j) pos[j] = pos0 + j;
    } else {
        pos[0] = pos0;
#pragma unroll
        for (int j = 1; j < NW; ++j) pos[j] = (pos[j - 1] + 1 == Mw) ? 0u : pos[j - 1] + 1;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            m[j] = et.mrow[pos[j]];
            bv[j] = et.ta.bw(pos[j]);
            kd[j] = et.ta.kdw(pos[j]);
        }
    }
    bool mis[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) mis[j] = live && ((x[j] ^ bv[j]) & m[j]) != 0;
    // participation: a chunk matches when none of its words mismatches
    bool p[NW];
    uint32_t hbits;  // the lane's header bits from chunk c0 on
    if (g == 1) {
        hbits = 0;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            p[j] = !mis[j];
            hbits |= (uint32_t)p[j] << j;
        }
    } else if (NW == 4 && g == 2) {
        // two chunks per lane (words 0-1 and 2-3)
        const bool pa = !(mis[0] || mis[1 % NW]), pb = !(mis[2 % NW] || mis[3 % NW]);
#pragma unroll
        for (int j = 0; j < NW; ++j) p[j] = j < 2 ? pa : pb;
        hbits = (uint32_t)pa | ((uint32_t)pb << 1);
    } else {
        const uint32_t q = g / NW;  // lanes per chunk
        bool any = false;
#pragma unroll
        for (int j = 0; j < NW; ++j) any = any || mis[j];
        const uint64_t bal = ballot(any);
        const uint32_t gs = lane & ~(q - 1u);
        const uint64_t qmask = (q >= 64) ? ~0ull : ((1ull << q) - 1ull);
        const bool pc = ((bal >> gs) & qmask) == 0;
#pragma unroll
        for (int j = 0; j < NW; ++j) p[j] = pc;
        hbits = (lane & (q - 1u)) == 0 ? (uint32_t)pc : 0u;
    }
    if constexpr (HDR) {
        // Two words per lane and W = 32: the sixteen lanes of a DPP row hold
        // one header word, since the step starts on a header-word boundary.
        // OR-ing their bits up the row and writing the word from its last
        // lane takes one LDS access per word instead of sixteen to the same
        // address (dense_gnn encode 7.7 -> 6.8 us; with four words per lane,
        // eight lanes to a word, the same OR measured no faster on the KV
        // pages or the llm_bf16 layers, so those keep one OR per lane).
        if (NW == 2 && g == 1) {
            uint32_t h = live ? hbits << (c0 & 31u) : 0u;
            h |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x111, 0xf, 0xf, false);
            h |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x112, 0xf, 0xf, false);
            h |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x114, 0xf, 0xf, false);
            h |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0x118, 0xf, 0xf, false);
            if ((lane & 15u) == 15u && h) atomicOr(&hdr[c0 >> 5], h);
        } else if (live && hbits) {
            atomicOr(&hdr[c0 >> 5], hbits << (c0 & 31u));
        }
    }
    // run masks of the lane's positions: one vector read per run
    uint32_t rr[RUNS > 0 ? RUNS : 1][NW];
    if constexpr (REGS) {
#pragma unroll
        for (int r = 0; r < RUNS; ++r)
#pragma unroll
            for (int j = 0; j < NW; ++j) rr[r][j] = et.r[r][j];
    } else if constexpr (MW4 && !UNI) {
#pragma unroll
        for (int r = 0; r < RUNS; ++r) load_vec<NW>(et.ta.r + (uint32_t)r * Mw + pos0, rr[r]);
    }
    uint32_t tot = 0;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        uint32_t e;
        if constexpr (REGS) {
            // at most three runs: their shifts are kd's upper bytes
            e = 0;
#pragma unroll
            for (int r = 0; r < RUNS; ++r) e |= (x[j] & rr[r][j]) >> ((kd[j] >> (8 * (r + 1))) & 31u);
        } else if constexpr (UNI) {
            e = extract_t<RUNS>(tu, 0, kd[j], x[j]);
        } else if constexpr (MW4) {
            e = 0;
#pragma unroll
            for (int r = 0; r < RUNS; ++r) e |= (x[j] & rr[r][j]) >> (et.ta.dw(r, pos[j], kd[j]) & 31u);
        } else {
            e = extract_t<RUNS>(et.ta, pos[j], kd[j], x[j]);
        }
        f[j] = p[j] ? e : x[j];
        size[j] = live ? (p[j] ? 32u - (kd[j] & 63u) : 32u) : 0u;
        tot += size[j];
    }
    return tot;
}

// Places one step's fields after the record's first `carry` payload bits (a
// wave scan of the lanes' widths gives each lane its offset) and advances
// carry by the step's total.
template <int NW>
__device__ __forceinline__ void or_fields(uint32_t* pay, uint32_t& carry, const uint32_t (&f)[NW],
                                          const uint32_t (&size)[NW], uint32_t tot) {
    const uint32_t incl = wave_incl_scan(tot);
    uint32_t off = carry + incl - tot;
    carry += lane_value(incl, kWave - 1);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        if (size[j]) {
            const uint32_t q = off >> 5, sh = off & 31u;
            atomicOr(&pay[q], f[j] << sh);
            if (sh + size[j] > 32) atomicOr(&pay[q + 1], f[j] >> (32 - sh));
        }
        off += size[j];
    }
}

// ---------------------------------------------------------------------------
// Tensors of at most kMaxTileWords words with 16-byte aligned source and
// slots: persistent workgroups, each taking a contiguous range of tensors,
// tables staged once in LDS, four words per lane per step (two for tensors of
// at most 128 words), and each step's words of the wave's next tensor in
// flight in the registers the current step has just consumed.  The record is
// assembled in LDS (header words, then the kept bits) and written with
// 16-byte stores; an incompressible tensor is copied from its source again.
// The range's bitmask bits are gathered in LDS and written once per word.
//
// Item placement: fixed slots (items.offsets == nullptr) or the packed cache
// layout, where the item goes to its offset once its length has been checked
// against the offsets.  SIZES: only the item lengths, rounded up to 16 bytes,
// are computed and written to sizes[] (no record buffer, no slot writes).
// headers != nullptr (at most 4 header words): the header words go to
// headers[t * hw ...] in GPU memory and the slot receives the payload only,
// which the record buffer then keeps 16-byte aligned after a 4-word header
// area.
// ---------------------------------------------------------------------------
template <int RUNS, bool UNI, bool MW4, int STAGE, bool SIZES>
__global__ __launch_bounds__(1024) void k_encode_small(Tables t, Geo geo, const uint8_t* __restrict__ src,
                                                      uint64_t n_tensors, uint8_t* __restrict__ slots,
                                                      uint32_t* __restrict__ bitmask, uint64_t* __restrict__ stored,
                                                      uint32_t buf_words, Items items, uint64_t* __restrict__ sizes,
                                                      uint32_t* err, uint32_t* __restrict__ headers) {
    extern __shared__ uint32_t smem[];
    // bitmask bits of the workgroup's tensors: set (compressed) and touched
    // (written at all), one bit per tensor from bit b0 % 32 of word 0
    __shared__ uint32_t bm_set[kEncBlockBitWords], bm_touched[kEncBlockBitWords];
    const uint32_t lane = lane_id();
    const uint32_t wib = uniform(threadIdx.x / kWave);
    const uint32_t Mw = geo.Mw;
    if (threadIdx.x < kEncBlockBitWords) bm_set[threadIdx.x] = bm_touched[threadIdx.x] = 0u;
    // LDS: [m row + per-position tables (not for uniform metadata)][wave buffers]
    const uint32_t rows = UNI ? 0u : 1u + tab_rows(RUNS);
    stage_table_image<dx_rows(RUNS)>(t, 0, rows, Mw, nullptr, 0, smem);
    __syncthreads();
    uint32_t* buf = smem + ((rows * Mw + 3u) & ~3u) + wib * buf_words;
    EncTabs<RUNS, UNI> et{};
    et.mrow = smem;
    et.ta = TabArrays{smem + Mw, smem + 2 * Mw, smem + 3 * Mw, smem + (3 + dx_rows(RUNS)) * Mw, Mw};
    if constexpr (UNI) {
        et.tu = load_uniform<RUNS>(t, Mw);
        et.mu = uniform(t.m[0]);
    }

    // STAGE 0: tensors of at most 128 words, two words per lane in one step
    // (four would leave half the lanes idle on a 512-byte row)
    constexpr int NW = STAGE == 0 ? 2 : 4;
    constexpr int kSt = STAGE == 0 ? 1 : STAGE;
    using Vec = std::conditional_t<NW == 4, u32x4, u32x2>;
    const uint32_t nw = (uint32_t)geo.n_words;
    const uint32_t nvec = nw / NW;
    const uint32_t hw = (uint32_t)geo.hdr_words;
    const uint32_t lg = geo.log2g;
    const uint32_t step_inc = (uint32_t)(NW * kWave) % Mw;
    // The workgroup takes tensors [b0, b1), its waves every wpb-th of them,
    // so that their bitmask bits gather in LDS: a bitmask word then takes one
    // store, or an atomic or two where neighbouring ranges share it (an
    // atomic per tensor, 32 to a word, cost 512-byte rows 2.4x the encode).
    const uint32_t wpb = blockDim.x / kWave;
    const uint64_t stride = wpb;
    const uint64_t per_block = (n_tensors + gridDim.x - 1) / gridDim.x;
    const uint64_t b0 = min((uint64_t)blockIdx.x * per_block, n_tensors);
    const uint64_t b1 = min(b0 + per_block, n_tensors);
    uint64_t ti = b0 + wib;

    // cur[s]: the lane's words of step s.  Once step s has taken them, the
    // same registers receive step s of the wave's next tensor, so the
    // prefetch costs no registers beyond one step's words.
    Vec cur[kSt];
    if (ti < b1) {
        const Vec* sv = reinterpret_cast<const Vec*>(src + ti * geo.L);
        static_for<kSt>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            const uint32_t i = lane + (uint32_t)r * kWave;
            if (i < nvec) cur[r] = __builtin_nontemporal_load(sv + i);
        });
    }
    for (; ti < b1; ti += stride) {
        const uint64_t tnext = ti + stride;
        const Vec* nxv = reinterpret_cast<const Vec*>(src + (tnext < b1 ? tnext : ti) * geo.L);
        // packed placement: this tensor's item span, needed once the record is built
        uint64_t item_a = 0, item_b = 0;
        if (!SIZES && items.offsets) {
            item_a = items.offsets[ti];
            item_b = items.offsets[ti + 1];
        }
        // zero the record buffer: header words, then the kept bits
        if constexpr (!SIZES) {
            u32x4* b4 = reinterpret_cast<u32x4*>(buf);
            for (uint32_t i = lane; i < (buf_words >> 2); i += kWave) b4[i] = u32x4{0u, 0u, 0u, 0u};
        }
        __builtin_amdgcn_wave_barrier();
        uint32_t* pay = buf + (headers ? 4u : hw);
        uint32_t carry = 0;
        uint32_t pos0 = UNI ? 0u : ((uint32_t)NW * lane) % Mw;
        static_for<kSt>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            const uint32_t lw0 = (uint32_t)s * (NW * kWave) + NW * lane;
            if ((uint32_t)s * (NW * kWave) >= nw) return;  // wave-uniform, and so for every later step
            const bool live = lw0 < nw;  // nw % 4 == 0: a live lane owns all its words
            const Vec xv = cur[s];
            if (tnext < b1 && live) cur[s] = __builtin_nontemporal_load(nxv + lane + (uint32_t)s * kWave);
            uint32_t x[NW];
#pragma unroll
            for (int j = 0; j < NW; ++j) x[j] = xv[j];
            uint32_t f[NW], size[NW];
            const uint32_t tot =
                encode_lane<NW, RUNS, UNI, MW4, !SIZES>(et, Mw, lg, live, pos0, x, buf, lw0 >> lg, f, size);
            if constexpr (SIZES)
                carry += wave_sum(tot);
            else
                or_fields(pay, carry, f, size, tot);
            if constexpr (!UNI) {
                pos0 += step_inc;
                if (pos0 >= Mw) pos0 -= Mw;
            }
        });
        __builtin_amdgcn_wave_barrier();
        const uint64_t R = 32ull * hw + carry;
        const uint32_t words = (uint32_t)((R + 31) / 32);
        const bool comp = 4ull * words < geo.L;
        const uint64_t item16 = ((comp ? 4ull * words : geo.L) + 15) & ~15ull;
        if constexpr (SIZES) {
            if (lane == 0) sizes[ti] = item16;
            continue;
        }
        u32x4* slot4 = reinterpret_cast<u32x4*>(slots + (items.offsets ? item_a : ti * geo.L));
        if (items.offsets && (item_b < item_a || item_b - item_a != item16 || item_b > items.bytes ||
                              (item_a & 15))) {
            // offsets that do not describe this tensor's item: write nothing
            latch_error(err, item_b > items.bytes ? kErrRange : kErrCorrupt);
            __builtin_amdgcn_wave_barrier();
            continue;
        }
        // header words to GPU memory (zero for a raw tensor) when they live there
        if (headers && lane < hw) headers[ti * hw + lane] = comp ? buf[lane] : 0u;
        if (comp) {
            // the record, or with headers in GPU memory its payload alone;
            // either fits the slot, a multiple of 16 bytes
            const uint32_t w4 = ((headers ? words - hw : words) + 3) >> 2;
            const u32x4* b4 = reinterpret_cast<const u32x4*>(headers ? pay : buf);
            for (uint32_t i = lane; i < w4; i += kWave) __builtin_nontemporal_store(b4[i], slot4 + i);
        } else {
            // the registers already hold the next tensor: copy this one again
            copy_words(reinterpret_cast<const uint32_t*>(src + ti * geo.L), reinterpret_cast<uint32_t*>(slot4), 0,
                       nw, true);
        }
        if (lane == 0) {
            const uint32_t j = (uint32_t)((ti >> 5) - (b0 >> 5)), bit = 1u << (ti & 31);
            atomicOr(&bm_touched[j], bit);
            if (comp) atomicOr(&bm_set[j], bit);
            if (stored) stored[ti] = comp ? 4ull * (headers ? words - hw : words) : geo.L;
        }
        __builtin_amdgcn_wave_barrier();
    }
    if constexpr (!SIZES) {
        __syncthreads();
        const uint32_t n_bw = b1 > b0 ? (uint32_t)(((b1 - 1) >> 5) - (b0 >> 5) + 1) : 0u;
        if (threadIdx.x < n_bw) {
            const uint32_t set = bm_set[threadIdx.x], touched = bm_touched[threadIdx.x];
            uint32_t* w = bitmask + (b0 >> 5) + threadIdx.x;
            if (touched == ~0u) {
                *w = set;  // every tensor of the word is this workgroup's
            } else {
                if (set) atomicOr(w, set);
                if (touched & ~set) atomicAnd(w, ~(touched & ~set));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Short launches from GPU memory to GPU memory: tensors of at most 1 KiB
// (one step of NW words per lane) and at most a few rows per CU.  A
// workgroup of 16 waves takes 32 consecutive tensors, two per wave, so that
// their bitmask bits fill exactly one bitmask word; nothing is staged: both
// rows' source words are loaded at once (range-checked buffer loads), and
// the table entries of the lanes' positions (or the wave-uniform words of
// uniform metadata) straight into registers.  Each record is assembled in
// its own LDS buffer as in k_encode_small and written with 16-byte stores;
// an incompressible tensor is stored from the registers that hold it.
// ---------------------------------------------------------------------------
// Rows per wave, measured on MI355X (16,384 rows of 512 bytes / of 1 KiB,
// header bits then still OR-ed one lane at a time): 2 rows (16 waves)
// 7.8-7.9 / 8.3-8.4 us, 4 rows (8 waves) 7.9-8.2 / 9.5 us, 8 rows (4 waves)
// 8.9-9.5 / 11.6 us.
constexpr uint32_t kEncRowWaves = 16, kEncRowsPerWave = 2;

template <int RUNS, bool UNI, int NW>
__global__ __launch_bounds__(kWave * kEncRowWaves) void k_encode_rows(Tables t, Geo geo,
                                                                     const uint8_t* __restrict__ src,
                                                                     uint64_t n_tensors, uint8_t* __restrict__ slots,
                                                                     uint32_t* __restrict__ bitmask,
                                                                     uint64_t* __restrict__ stored,
                                                                     uint32_t buf_words) {
    extern __shared__ uint32_t smem[];
    __shared__ uint32_t bm_set, bm_touched;
    using Vec = std::conditional_t<NW == 4, u32x4, u32x2>;
    const uint32_t lane = lane_id();
    const uint32_t wib = uniform(threadIdx.x / kWave);
    const uint64_t b0 = (uint64_t)blockIdx.x * (kEncRowWaves * kEncRowsPerWave);
    const uint64_t t0 = b0 + (uint64_t)wib * kEncRowsPerWave;
    const uint32_t nw = (uint32_t)geo.n_words;
    const uint32_t Mw = geo.Mw;
    if (threadIdx.x == 0) bm_set = bm_touched = 0u;
    // both rows' words (lanes past a row, or a row past the launch, read zeros)
    Vec xv[kEncRowsPerWave];
    static_for<kEncRowsPerWave>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const bool in = t0 + r < n_tensors;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(src + (in ? (t0 + r) * geo.L : 0)), (short)0, (int)(in ? geo.L : 0), 0x00020000);
        if constexpr (NW == 4)
            xv[r] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(16 * lane), 0, 2);
        else
            xv[r] = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(8 * lane), 0, 2);
    });
    std::conditional_t<UNI, EncTabs<RUNS, true>, EncRegs<UNI ? 0 : RUNS, NW>> et;
    if constexpr (UNI) {
        et = enc_tabs_global<RUNS, true>(t, Mw);
    } else {
        // a period of at least a step's words needs no wrap (and no division)
        const uint32_t p0 = (uint32_t)NW * lane;
        if (Mw >= (uint32_t)NW * kWave)
            et.load(t, Mw, p0);
        else
            et.load(t, Mw, p0 % Mw);
    }
    __syncthreads();
    const uint32_t hw = (uint32_t)geo.hdr_words;
    const uint32_t lw0 = (uint32_t)NW * lane;
    const bool live = lw0 < nw;  // nw % 4 == 0: a live lane owns all its words
    static_for<kEncRowsPerWave>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        const uint64_t ti = t0 + r;
        if (ti >= n_tensors) return;
        uint32_t* buf = smem + (wib * kEncRowsPerWave + r) * buf_words;
        u32x4* b4 = reinterpret_cast<u32x4*>(buf);
        for (uint32_t i = lane; i < (buf_words >> 2); i += kWave) b4[i] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_wave_barrier();
        uint32_t x[NW];
#pragma unroll
        for (int j = 0; j < NW; ++j) x[j] = xv[r][j];
        uint32_t f[NW], size[NW];
        // (the positions only feed the table reads, which EncRegs has done)
        const uint32_t tot = encode_lane<NW, RUNS, UNI, true, true>(et, Mw, geo.log2g, live, 0u, x, buf,
                                                                    lw0 >> geo.log2g, f, size);
        uint32_t carry = 0;
        or_fields(buf + hw, carry, f, size, tot);
        __builtin_amdgcn_wave_barrier();
        const uint64_t R = 32ull * hw + carry;
        const uint32_t words = (uint32_t)((R + 31) / 32);
        const bool comp = 4ull * words < geo.L;
        uint8_t* slot = slots + ti * geo.L;
        if (comp) {
            const uint32_t w4 = (words + 3) >> 2;
            for (uint32_t i = lane; i < w4; i += kWave)
                __builtin_nontemporal_store(b4[i], reinterpret_cast<u32x4*>(slot) + i);
        } else if (live) {
            __builtin_nontemporal_store(xv[r], reinterpret_cast<Vec*>(slot) + lane);
        }
        if (lane == 0) {
            const uint32_t bit = 1u << (uint32_t)(ti - b0);
            atomicOr(&bm_touched, bit);
            if (comp) atomicOr(&bm_set, bit);
            if (stored) stored[ti] = comp ? 4ull * words : geo.L;
        }
    });
    __syncthreads();
    if (threadIdx.x == 0) {
        // the workgroup's 32 tensors are one bitmask word (b0 is a multiple of 32)
        const uint32_t set = bm_set, touched = bm_touched;
        uint32_t* w = bitmask + (b0 >> 5);
        if (touched == ~0u) {
            *w = set;
        } else {
            if (set) atomicOr(w, set);
            if (touched & ~set) atomicAnd(w, ~(touched & ~set));
        }
    }
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
// Tensors longer than one tile whose source is in device memory (16-byte
// aligned): start bits without look-back.  A look-back chain moves its
// inclusive prefix by at most one wave's window of tiles per memory round
// trip, which holds an HBM-resident encode far below the memory bound; a
// second read of the source costs less.  k_enc_group_bits: one wave per group
// of TPG tiles runs the match test over the group's words and writes the
// group's payload bits; launch_group_scan turns them into each group's start
// bit.  k_encode_groups: one wave per group encodes its tiles in order, four
// words per lane per step (each step's words of the next tile are loaded as
// the step consumes the current one), and writes each tile's header words
// and the payload words whose last bit falls in it.  The bits of the previous
// tile that share its first word are carried over in a register within the
// group and rebuilt from the source at the group's first tile.
// ---------------------------------------------------------------------------
template <int RUNS, bool UNI, bool MW4, uint32_t TPG>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void k_enc_group_bits(Tables t, Geo geo,
                                                                           const uint8_t* __restrict__ src,
                                                                           uint64_t n_tensors, uint64_t* bits) {
    constexpr uint32_t kBatch = 4;  // steps whose loads are issued together
    const uint32_t lane = lane_id();
    const uint64_t gpt = tile_groups(geo.tiles_per_tensor, TPG);
    const uint64_t group = (uint64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x / kWave);
    if (group >= n_tensors * gpt) return;
    const uint64_t ti = group / gpt;
    const uint64_t w0 = (group - ti * gpt) * TPG * kLongTileWordsEncode;
    const uint32_t nw = (uint32_t)min((uint64_t)TPG * kLongTileWordsEncode, geo.n_words - w0);
    const uint32_t n4 = nw >> 2;
    const u32x4* x4 = reinterpret_cast<const u32x4*>(src + ti * geo.L) + (w0 >> 2);
    const EncTabs<RUNS, UNI> et = enc_tabs_global<RUNS, UNI>(t, geo.Mw);
    const uint32_t Mw = geo.Mw;
    const uint32_t step_inc = (uint32_t)(4 * kWave) % Mw;
    uint32_t pos0 = UNI ? 0u : (uint32_t)((w0 + 4 * lane) % Mw);
    const uint32_t steps = (n4 + kWave - 1) / kWave;
    uint32_t acc = 0;
    for (uint32_t s0 = 0; s0 < steps; s0 += kBatch) {
        u32x4 v[kBatch];
        static_for<kBatch>([&](auto uc) {
            constexpr uint32_t u = decltype(uc)::value;
            // past the group's end: its last vector again (all loads in flight together)
            const uint32_t i = min((s0 + u) * kWave + lane, n4 - 1);
            v[u] = __builtin_nontemporal_load(x4 + i);
        });
        static_for<kBatch>([&](auto uc) {
            constexpr uint32_t u = decltype(uc)::value;
            if (s0 + u >= steps) return;  // wave-uniform
            const bool live = (s0 + u) * kWave + lane < n4;
            const uint32_t x[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
            uint32_t f[4], size[4];
            acc += encode_lane<4, RUNS, UNI, MW4, false>(et, Mw, geo.log2g, live, pos0, x, nullptr, 0, f, size);
            if constexpr (!UNI) {
                pos0 += step_inc;
                if (pos0 >= Mw) pos0 -= Mw;
            }
        });
    }
    const uint32_t tot = wave_sum(acc);
    if (lane == 0) bits[group] = tot;
}

template <int RUNS, bool UNI, bool MW4, uint32_t TPG>
__global__ __launch_bounds__(kWave * kWavesPerBlock) void k_encode_groups(Tables t, Geo geo,
                                                                          const uint8_t* __restrict__ src,
                                                                          uint64_t n_tensors,
                                                                          uint8_t* __restrict__ slots,
                                                                          const uint64_t* __restrict__ starts,
                                                                          uint64_t* __restrict__ totals,
                                                                          uint32_t lds_words) {
    extern __shared__ uint32_t smem[];
    constexpr uint32_t TW = kLongTileWordsEncode;
    constexpr uint32_t kSteps = TW / (4 * kWave);
    const uint32_t lane = lane_id();
    const uint32_t wib = uniform(threadIdx.x / kWave);
    const uint64_t gpt = tile_groups(geo.tiles_per_tensor, TPG);
    const uint64_t group = (uint64_t)blockIdx.x * kWavesPerBlock + wib;
    if (group >= n_tensors * gpt) return;
    const uint64_t ti = group / gpt;
    const uint64_t tile0 = (group - ti * gpt) * TPG;
    const uint32_t ntiles = (uint32_t)min((uint64_t)TPG, geo.tiles_per_tensor - tile0);
    const uint32_t* x = reinterpret_cast<const uint32_t*>(src + ti * geo.L);
    const u32x4* x4 = reinterpret_cast<const u32x4*>(x);
    uint32_t* slot = reinterpret_cast<uint32_t*>(slots + ti * geo.L);
    // LDS of the wave: 64 header words, then the tile's payload bits
    uint32_t* hdr = smem + wib * lds_words;
    uint32_t* pay = hdr + 64;
    const EncTabs<RUNS, UNI> et = enc_tabs_global<RUNS, UNI>(t, geo.Mw);
    const uint32_t Mw = geo.Mw, lg = geo.log2g;
    const uint32_t step_inc = (uint32_t)(4 * kWave) % Mw;

    uint64_t S = uniform64(starts[group]);
    uint64_t w0 = tile0 * TW;
    // bits [32 * (S >> 5), S) of the record: the end of the previous tile
    uint32_t tail = 0;
    if (tile0 > 0 && (S & 31)) tail = bits_before_tile<RUNS>(t, geo, x, w0, (uint32_t)(S & 31));

    // Tile k's words are in cur; the next tile's are loaded into nxt as the
    // tile starts, with range-checked buffer loads: every tile issues the same
    // number, and those past the next tile (all of them when the group has no
    // next tile) return zero without touching memory.  The arrays swap roles
    // from tile to tile, so no register that a load in flight writes is
    // copied (a copy waits for its load).
    u32x4 buf_a[kSteps], buf_b[kSteps];
    {
        const uint32_t n4 = (uint32_t)min((uint64_t)TW, geo.n_words - w0) >> 2;
        static_for<kSteps>([&](auto sc) {
            constexpr uint32_t s = decltype(sc)::value;
            if (s * kWave + lane < n4) buf_a[s] = __builtin_nontemporal_load(x4 + (w0 >> 2) + s * kWave + lane);
        });
    }
    auto one_tile = [&](u32x4(&cur)[kSteps], u32x4(&nxt)[kSteps], uint32_t k) __attribute__((always_inline)) {
        const uint32_t nw = (uint32_t)min((uint64_t)TW, geo.n_words - w0);
        const uint64_t wn = w0 + TW;
        const uint32_t nn4 = k + 1 < ntiles ? (uint32_t)min((uint64_t)TW, geo.n_words - wn) >> 2 : 0u;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(x4 + (k + 1 < ntiles ? wn >> 2 : 0)), (short)0, (int)(16 * nn4), 0x00020000);
        u32x4* z4 = reinterpret_cast<u32x4*>(hdr);
        for (uint32_t i = lane; i < (lds_words >> 2); i += kWave) z4[i] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_wave_barrier();
        static_for<kSteps>([&](auto sc) {
            constexpr uint32_t s = decltype(sc)::value;
            nxt[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(16 * (s * kWave + lane)), 0, 2);
        });
        uint32_t carry = 0;
        uint32_t pos0 = UNI ? 0u : (uint32_t)((w0 + 4 * lane) % Mw);
        static_for<kSteps>([&](auto sc) {
            constexpr uint32_t s = decltype(sc)::value;
            if (s * 4 * kWave >= nw) return;  // wave-uniform, and so for every later step
            const uint32_t lw0 = s * 4 * kWave + 4 * lane;
            const bool live = lw0 < nw;
            const u32x4 xv = cur[s];
            const uint32_t x[4] = {xv[0], xv[1], xv[2], xv[3]};
            uint32_t f[4], size[4];
            const uint32_t tot = encode_lane<4, RUNS, UNI, MW4, true>(et, Mw, lg, live, pos0, x, hdr, lw0 >> lg, f, size);
            or_fields(pay, carry, f, size, tot);
            if constexpr (!UNI) {
                pos0 += step_inc;
                if (pos0 >= Mw) pos0 -= Mw;
            }
        });
        __builtin_amdgcn_wave_barrier();
        const uint64_t E = S + carry;
        const bool last = tile0 + k == geo.tiles_per_tensor - 1;
        // the tile's header words (always inside the slot)
        const uint64_t hw0 = (w0 >> lg) >> 5;
        const uint32_t hw_t = ((nw >> lg) + 31) / 32;
        for (uint32_t j = lane; j < hw_t; j += kWave) slot[hw0 + j] = hdr[j];
        // Payload words whose last bit lies in [S, E); the tensor's last tile
        // also writes the final partial word, zero padded.  A record longer
        // than the slot is cut off here and replaced by the raw tensor later.
        // Word q0 + i is bits [32 i, 32 i + 32) of the tile's payload shifted
        // up by r, below them the open bits of the previous tile: with those
        // bits in the word before the payload (shifted to its top), word i is
        // a funnel shift of two neighbouring LDS words, 16-byte stores from
        // the first aligned word on.
        const uint64_t q0 = S >> 5;
        uint64_t q1 = E >> 5;
        if (last && (E & 31)) q1 += 1;
        q1 = min(q1, geo.n_words);
        const uint32_t r = (uint32_t)(S & 31);
        const uint32_t sh = (32u - r) & 31u;
        if (lane == 0) pay[-1] = r ? tail << (32u - r) : 0u;
        __builtin_amdgcn_wave_barrier();
        const uint32_t* P = r ? pay - 1 : pay;
        const uint32_t n = q1 > q0 ? (uint32_t)(q1 - q0) : 0u;
        const uint32_t head = min((4u - (uint32_t)(q0 & 3)) & 3u, n);
        const uint32_t nv = (n - head) >> 2;
        const uint32_t rest = head + 4 * nv;  // words [rest, n) after the last vector
        uint32_t* sq = slot + q0;
        if (lane < head) {
            sq[lane] = funnel(P[lane + 1], P[lane], sh);
        } else if (lane >= 4 && lane - 4 < n - rest) {
            const uint32_t i = rest + lane - 4;
            sq[i] = funnel(P[i + 1], P[i], sh);
        }
        for (uint32_t v = lane; v < nv; v += kWave) {
            const uint32_t i = head + 4 * v;
            u32x4 w;
    #pragma unroll
            for (uint32_t c = 0; c < 4; ++c) w[c] = funnel(P[i + c + 1], P[i + c], sh);
            *reinterpret_cast<u32x4*>(sq + i) = w;
        }
        // bits [32 * (E >> 5), E) for the next tile
        const uint32_t iE = (uint32_t)((E >> 5) - q0);
        tail = uniform(funnel(P[iE + 1], P[iE], sh));
        if (last && lane == 0) totals[ti] = E;
        S = E;
        w0 = wn;
        __builtin_amdgcn_wave_barrier();
    };
    for (uint32_t k = 0; k < ntiles; k += 2) {
        one_tile(buf_a, buf_b, k);
        if (k + 1 < ntiles) one_tile(buf_b, buf_a, k + 1);
    }
}

template <int RUNS, bool UNI, bool MW4>
static hipError_t launch_encode_groups_s(const Tables& t, const Geo& geo, const void* src, uint64_t n_tensors,
                                         void* slots, const LookBack& lb, hipStream_t s) {
    constexpr uint32_t TPG = kEncodeTilesPerGroupHbm;
    const uint64_t groups = n_tensors * tile_groups(geo.tiles_per_tensor, TPG);
    uint64_t* starts = reinterpret_cast<uint64_t*>(lb.status);  // one word per group
    const dim3 grid((uint32_t)((groups + kWavesPerBlock - 1) / kWavesPerBlock));
    const dim3 block(kWave * kWavesPerBlock);
    const uint8_t* sr = static_cast<const uint8_t*>(src);
    hipLaunchKernelGGL((k_enc_group_bits<RUNS, UNI, MW4, TPG>), grid, block, 0, s, t, geo, sr, n_tensors, starts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_group_scan(n_tensors, tile_groups(geo.tiles_per_tensor, TPG), 32ull * geo.hdr_words, starts, s);
    if (e != hipSuccess) return e;
    // 64 header words, the tile's payload and the zero words after it
    const uint32_t lds_words = 64 + kLongTileWordsEncode + 8;
    hipLaunchKernelGGL((k_encode_groups<RUNS, UNI, MW4, TPG>), grid, block, (size_t)lds_words * 4 * kWavesPerBlock, s,
                       t, geo, sr, n_tensors, static_cast<uint8_t*>(slots), starts, lb.totals, lds_words);
    return hipGetLastError();
}

template <int RUNS>
static hipError_t launch_encode_groups(const Tables& t, const Geo& geo, bool uniform_meta, const void* src,
                                       uint64_t n_tensors, void* slots, const LookBack& lb, hipStream_t s) {
    if (uniform_meta) return launch_encode_groups_s<RUNS, true, false>(t, geo, src, n_tensors, slots, lb, s);
    if (geo.Mw % 4 == 0) return launch_encode_groups_s<RUNS, false, true>(t, geo, src, n_tensors, slots, lb, s);
    return launch_encode_groups_s<RUNS, false, false>(t, geo, src, n_tensors, slots, lb, s);
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

// LDS k_encode_small shares per workgroup (tables) and needs per wave (record
// buffer); false when the tables do not fit.
static bool small_encode_lds(const Geo& geo, int runs, bool uni, uint32_t* buf_words, size_t* head,
                             size_t* wave) {
    // header words (at least a 4-word area, so that a payload written
    // without its header stays 16-byte aligned) + kept bits + 2 spare words,
    // rounded to 16 bytes
    const uint32_t hdr_area = geo.hdr_words < 4 ? 4u : (uint32_t)geo.hdr_words;
    *buf_words = (hdr_area + (uint32_t)geo.n_words + 2 + 3) & ~3u;
    const uint64_t tab = uni ? 0 : (uint64_t)(1 + tab_rows(runs)) * geo.Mw * 4;
    if (tab > kMaxLdsTableBytes) return false;
    *head = (size_t)((tab + 15) & ~15ull);
    *wave = (size_t)*buf_words * 4;
    return true;
}

// Extra arguments of the packed-cache modes (defaults: fixed slots).
struct SmallArgs {
    Items items{nullptr, 0};
    uint64_t* sizes = nullptr;
    uint32_t* err = nullptr;
    uint32_t* headers = nullptr;
};

template <int RUNS, bool UNI, bool MW4, int S, bool SIZES>
static hipError_t launch_encode_small_s(const Tables& t, const Geo& geo, const void* src, uint64_t n_tensors,
                                        void* slots, uint32_t* bitmask, uint64_t* stored, uint32_t cu_count,
                                        size_t head, size_t wave, uint32_t buf_words, const SmallArgs& xa,
                                        hipStream_t s, bool* launched) {
    const void* fn = reinterpret_cast<const void*>(&k_encode_small<RUNS, UNI, MW4, S, SIZES>);
    PersistentPlan plan;
    *launched = false;
    if (!plan_persistent(fn, head, SIZES ? 0 : wave, cu_count, n_tensors, &plan)) return hipSuccess;
    // a workgroup's tensors must span at most kEncBlockBitWords bitmask words
    const uint64_t per_block = (n_tensors + plan.blocks - 1) / plan.blocks;
    if (per_block + 31 > 32ull * kEncBlockBitWords) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_encode_small<RUNS, UNI, MW4, S, SIZES>), dim3(plan.blocks), dim3(kWave * plan.wpb),
                       plan.shm, s, t, geo, static_cast<const uint8_t*>(src), n_tensors,
                       static_cast<uint8_t*>(slots), bitmask, stored, SIZES ? 0u : buf_words, xa.items, xa.sizes,
                       xa.err, xa.headers);
    *launched = true;
    return hipGetLastError();
}

template <int RUNS, bool UNI, bool SIZES>
static hipError_t launch_encode_small(const Tables& t, const Geo& geo, const void* src, uint64_t n_tensors,
                                      void* slots, uint32_t* bitmask, uint64_t* stored, uint32_t cu_count,
                                      size_t head, size_t wave, uint32_t buf_words, const SmallArgs& xa,
                                      hipStream_t s, bool* launched) {
    const uint32_t stage = (uint32_t)((geo.n_words + 4 * kWave - 1) / (4 * kWave));
    const bool mw4 = geo.Mw % 4 == 0;
#define IBP_ENC_SMALL(S)                                                                                        \
    return mw4 ? launch_encode_small_s<RUNS, UNI, true, S, SIZES>(t, geo, src, n_tensors, slots, bitmask,       \
                                                                  stored, cu_count, head, wave, buf_words, xa,  \
                                                                  s, launched)                                  \
               : launch_encode_small_s<RUNS, UNI, false, S, SIZES>(t, geo, src, n_tensors, slots, bitmask,      \
                                                                   stored, cu_count, head, wave, buf_words, xa, \
                                                                   s, launched)
    if (geo.n_words <= 2 * kWave) IBP_ENC_SMALL(0);
    if (stage <= 1) IBP_ENC_SMALL(1);
    if (stage <= 2) IBP_ENC_SMALL(2);
    if (stage <= 4) IBP_ENC_SMALL(4);
    IBP_ENC_SMALL(8);
#undef IBP_ENC_SMALL
}

// Single-tile tensors of at most 1 KiB encoded from GPU memory into GPU
// memory, 16-byte aligned, at most three runs per position unless the
// metadata is uniform, and at most 128 rows per CU: k_encode_rows.  0 sends
// every call to the persistent kernel.
#ifndef IBP_ENCODE_ROWS
#define IBP_ENCODE_ROWS 1
#endif

static bool encode_rows(const Geo& geo, int runs, bool uni, uint64_t n_tensors, uint32_t cu_count) {
    return IBP_ENCODE_ROWS && geo.src_in_hbm && geo.dst_in_hbm && geo.aligned16 && geo.n_words <= 4 * kWave &&
           (uni || (runs <= 3 && geo.Mw % 4 == 0)) && n_tensors <= 128ull * cu_count;
}

template <int RUNS, bool UNI>
static hipError_t launch_encode_rows(const Tables& t, const Geo& geo, const void* src, uint64_t n_tensors,
                                     void* slots, uint32_t* bitmask, uint64_t* stored, uint32_t buf_words,
                                     hipStream_t s) {
    if constexpr (!UNI && RUNS > 3) {
        return hipErrorInvalidValue;
    } else {
        constexpr uint32_t rows = kEncRowWaves * kEncRowsPerWave;
        const dim3 grid((uint32_t)((n_tensors + rows - 1) / rows));
        const size_t shm = (size_t)rows * buf_words * 4;
        if (geo.n_words <= 2 * kWave)
            hipLaunchKernelGGL((k_encode_rows<RUNS, UNI, 2>), grid, dim3(kWave * kEncRowWaves), shm, s, t, geo,
                               static_cast<const uint8_t*>(src), n_tensors, static_cast<uint8_t*>(slots), bitmask,
                               stored, buf_words);
        else
            hipLaunchKernelGGL((k_encode_rows<RUNS, UNI, 4>), grid, dim3(kWave * kEncRowWaves), shm, s, t, geo,
                               static_cast<const uint8_t*>(src), n_tensors, static_cast<uint8_t*>(slots), bitmask,
                               stored, buf_words);
        return hipGetLastError();
    }
}

template <int RUNS>
static hipError_t launch_encode_r(const Tables& t, const Geo& geo, bool uniform_meta, const void* src,
                                  uint64_t n_tensors, void* slots, uint32_t* bitmask, uint64_t* stored,
                                  const LookBack* lb, uint32_t cu_count, hipStream_t s) {
    const uint32_t lds_words = 64 + geo.tile_words + 8;
    if (geo.tiles_per_tensor == 1) {
        uint32_t buf_words = 0;
        size_t head = 0, wave = 0;
        if (geo.aligned16 && small_encode_lds(geo, RUNS, uniform_meta, &buf_words, &head, &wave)) {
            if (encode_rows(geo, RUNS, uniform_meta, n_tensors, cu_count))
                return uniform_meta ? launch_encode_rows<RUNS, true>(t, geo, src, n_tensors, slots, bitmask, stored,
                                                                     buf_words, s)
                                    : launch_encode_rows<RUNS, false>(t, geo, src, n_tensors, slots, bitmask,
                                                                      stored, buf_words, s);
            bool launched = false;
            const SmallArgs xa;
            const hipError_t e =
                uniform_meta ? launch_encode_small<RUNS, true, false>(t, geo, src, n_tensors, slots, bitmask, stored,
                                                                      cu_count, head, wave, buf_words, xa, s,
                                                                      &launched)
                             : launch_encode_small<RUNS, false, false>(t, geo, src, n_tensors, slots, bitmask,
                                                                       stored, cu_count, head, wave, buf_words, xa,
                                                                       s, &launched);
            if (e != hipSuccess || launched) return e;
        }
        return launch_encode_t<false>(t, geo, RUNS, src, n_tensors, slots, bitmask, stored, LookBack{}, lds_words,
                                      s);
    }
    hipError_t e = encode_two_pass(geo)
                       ? launch_encode_groups<RUNS>(t, geo, uniform_meta, src, n_tensors, slots, *lb, s)
                       : launch_encode_t<true>(t, geo, RUNS, src, n_tensors, slots, bitmask, stored, *lb, lds_words, s);
    if (e != hipSuccess) return e;
    uint64_t per = (geo.n_words + 256ull * 64 - 1) / (256ull * 64);  // ~64 words per thread
    if (per > 1024) per = 1024;
    const uint32_t bpt = (uint32_t)(per ? per : 1);
    hipLaunchKernelGGL(k_encode_finalize, dim3((uint32_t)(n_tensors * bpt)), dim3(256), 0, s, geo,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(slots), bitmask, stored,
                       lb->totals, bpt);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Item offsets of the packed cache: offsets[1..n] hold the item sizes and are
// turned into their inclusive prefix sums in place (offsets[0] <- 0).  One
// wave per block of kScanBlock sizes (eight consecutive per lane); blocks
// take dynamic tickets and chain their totals by decoupled look-back.  Items
// are at most 8 KiB, so a block's total fits in 32 bits.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scan_sizes(uint64_t* __restrict__ offsets, uint64_t n, LookBack lb) {
    const uint32_t lane = lane_id();
    uint32_t tk = 0;
    if (lane == 0) tk = atomicAdd(lb.ticket, 1u);
    const uint64_t blk = uniform(tk);
    const uint64_t n_blocks = (n + kScanBlock - 1) / kScanBlock;
    if (blk >= n_blocks) return;
    uint64_t* sz = offsets + 1;
    const uint64_t i0 = blk * kScanBlock + (uint64_t)lane * kScanPerLane;
    uint32_t v[kScanPerLane];
    uint32_t run = 0;
#pragma unroll
    for (uint32_t j = 0; j < kScanPerLane; ++j) {
        run += (i0 + j < n) ? (uint32_t)sz[i0 + j] : 0u;
        v[j] = run;
    }
    const uint32_t incl = wave_incl_scan(run);
    const uint32_t agg = lane_value(incl, kWave - 1);
    const uint64_t base = lookback_exclusive(lb.status, 0, blk, agg, 0, lb.epoch, lb.err);
    const uint64_t pre = base + (incl - run);
#pragma unroll
    for (uint32_t j = 0; j < kScanPerLane; ++j)
        if (i0 + j < n) sz[i0 + j] = pre + v[j];
    if (blk == 0 && lane == 0) offsets[0] = 0;
}

uint64_t scan_waves(uint64_t n) {
    const uint64_t n_blocks = (n + kScanBlock - 1) / kScanBlock;
    return ((n_blocks + kWavesPerBlock - 1) / kWavesPerBlock) * kWavesPerBlock;
}

hipError_t launch_scan_sizes(uint64_t* offsets, uint64_t n, const LookBack& lb, hipStream_t s) {
    if (n == 0) return launch_fill_u32(reinterpret_cast<uint32_t*>(offsets), 2, 0, s);
    const uint64_t waves = scan_waves(n);
    hipLaunchKernelGGL(k_scan_sizes, dim3((uint32_t)(waves / kWavesPerBlock)), dim3(kWave * kWavesPerBlock), 0, s,
                       offsets, n, lb);
    return hipGetLastError();
}

// Packed-cache entry points: the persistent small-tensor kernel in its
// sizes-only or packed-placement mode.
template <int RUNS>
static hipError_t launch_packed_r(const Tables& t, const Geo& geo, bool uniform_meta, bool sizes_only,
                                  const void* src, uint64_t n_tensors, void* dst, uint32_t* bitmask,
                                  const SmallArgs& xa, uint32_t cu_count, hipStream_t s) {
    uint32_t buf_words = 0;
    size_t head = 0, wave = 0;
    if (geo.tiles_per_tensor != 1 || !geo.aligned16 || !small_encode_lds(geo, RUNS, uniform_meta, &buf_words, &head, &wave))
        return hipErrorInvalidValue;
    bool launched = false;
    hipError_t e;
    if (sizes_only)
        e = uniform_meta ? launch_encode_small<RUNS, true, true>(t, geo, src, n_tensors, nullptr, nullptr, nullptr,
                                                                 cu_count, head, wave, buf_words, xa, s, &launched)
                         : launch_encode_small<RUNS, false, true>(t, geo, src, n_tensors, nullptr, nullptr, nullptr,
                                                                  cu_count, head, wave, buf_words, xa, s, &launched);
    else
        e = uniform_meta ? launch_encode_small<RUNS, true, false>(t, geo, src, n_tensors, dst, bitmask, nullptr,
                                                                  cu_count, head, wave, buf_words, xa, s, &launched)
                         : launch_encode_small<RUNS, false, false>(t, geo, src, n_tensors, dst, bitmask, nullptr,
                                                                   cu_count, head, wave, buf_words, xa, s,
                                                                   &launched);
    if (e != hipSuccess) return e;
    return launched ? hipSuccess : hipErrorInvalidValue;
}

static hipError_t launch_packed(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta, bool sizes_only,
                                const void* src, uint64_t n_tensors, void* dst, uint32_t* bitmask,
                                const SmallArgs& xa, uint32_t cu_count, hipStream_t s) {
    if (n_tensors == 0) return hipSuccess;
#define IBP_PK(R) return launch_packed_r<R>(t, geo, uniform_meta, sizes_only, src, n_tensors, dst, bitmask, xa, cu_count, s)
    switch (runs_bucket(runs)) {
        case 0: IBP_PK(0);
        case 1: IBP_PK(1);
        case 2: IBP_PK(2);
        case 3: IBP_PK(3);
        case 4: IBP_PK(4);
        case 8: IBP_PK(8);
        default: IBP_PK(16);
    }
#undef IBP_PK
}

bool split_supported(const Geo& geo, uint32_t runs, bool uniform_meta) {
    return geo.hdr_words <= kMaxSplitHeaderWords && packed_supported(geo, runs, uniform_meta);
}

template <int RUNS>
static hipError_t launch_encode_split_r(const Tables& t, const Geo& geo, bool uniform_meta, const void* src,
                                        uint64_t n_tensors, void* slots, uint32_t* headers, uint32_t* bitmask,
                                        uint64_t* stored, uint32_t cu_count, hipStream_t s) {
    uint32_t buf_words = 0;
    size_t head = 0, wave = 0;
    if (!small_encode_lds(geo, RUNS, uniform_meta, &buf_words, &head, &wave)) return hipErrorInvalidValue;
    SmallArgs xa;
    xa.headers = headers;
    bool launched = false;
    const hipError_t e =
        uniform_meta ? launch_encode_small<RUNS, true, false>(t, geo, src, n_tensors, slots, bitmask, stored, cu_count,
                                                              head, wave, buf_words, xa, s, &launched)
                     : launch_encode_small<RUNS, false, false>(t, geo, src, n_tensors, slots, bitmask, stored,
                                                               cu_count, head, wave, buf_words, xa, s, &launched);
    if (e != hipSuccess) return e;
    return launched ? hipSuccess : hipErrorInvalidValue;
}

hipError_t launch_encode_split(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta, const void* src,
                               uint64_t n_tensors, void* slots, uint32_t* headers, uint32_t* bitmask,
                               uint64_t* stored, uint32_t cu_count, hipStream_t s) {
    if (n_tensors == 0) return hipSuccess;
#define IBP_SP(R) return launch_encode_split_r<R>(t, geo, uniform_meta, src, n_tensors, slots, headers, bitmask, stored, cu_count, s)
    switch (runs_bucket(runs)) {
        case 0: IBP_SP(0);
        case 1: IBP_SP(1);
        case 2: IBP_SP(2);
        case 3: IBP_SP(3);
        case 4: IBP_SP(4);
        case 8: IBP_SP(8);
        default: IBP_SP(16);
    }
#undef IBP_SP
}

bool packed_supported(const Geo& geo, uint32_t runs, bool uniform_meta) {
    uint32_t buf_words = 0;
    size_t head = 0, wave = 0;
    return geo.tiles_per_tensor == 1 && geo.aligned16 &&
           small_encode_lds(geo, (int)runs_bucket(runs), uniform_meta, &buf_words, &head, &wave);
}

hipError_t launch_item_sizes(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta, const void* src,
                             uint64_t n_tensors, uint64_t* sizes, uint32_t cu_count, hipStream_t s) {
    SmallArgs xa;
    xa.sizes = sizes;
    return launch_packed(t, geo, runs, uniform_meta, true, src, n_tensors, nullptr, nullptr, xa, cu_count, s);
}

hipError_t launch_encode_packed(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta,
                                const void* src, uint64_t n_tensors, void* dst, const Items& items,
                                uint32_t* bitmask, uint32_t* err, uint32_t cu_count, hipStream_t s) {
    SmallArgs xa;
    xa.items = items;
    xa.err = err;
    return launch_packed(t, geo, runs, uniform_meta, false, src, n_tensors, dst, bitmask, xa, cu_count, s);
}

hipError_t launch_encode(const Tables& t, const Geo& geo, uint32_t runs, bool uniform_meta, const void* src,
                         uint64_t n_tensors, void* slots, uint32_t* bitmask, uint64_t* stored, const LookBack* lb,
                         uint32_t cu_count, hipStream_t s) {
    if (n_tensors == 0) return hipSuccess;
    switch (runs_bucket(runs)) {
        case 0: return launch_encode_r<0>(t, geo, uniform_meta, src, n_tensors, slots, bitmask, stored, lb, cu_count, s);
        case 1: return launch_encode_r<1>(t, geo, uniform_meta, src, n_tensors, slots, bitmask, stored, lb, cu_count, s);
        case 2: return launch_encode_r<2>(t, geo, uniform_meta, src, n_tensors, slots, bitmask, stored, lb, cu_count, s);
        case 3: return launch_encode_r<3>(t, geo, uniform_meta, src, n_tensors, slots, bitmask, stored, lb, cu_count, s);
        case 4: return launch_encode_r<4>(t, geo, uniform_meta, src, n_tensors, slots, bitmask, stored, lb, cu_count, s);
        case 8: return launch_encode_r<8>(t, geo, uniform_meta, src, n_tensors, slots, bitmask, stored, lb, cu_count, s);
        default: return launch_encode_r<16>(t, geo, uniform_meta, src, n_tensors, slots, bitmask, stored, lb, cu_count, s);
    }
}

}  // namespace ibp
