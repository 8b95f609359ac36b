// ibp_meta.hip -- step 1 of Invariant Bit Packing on gfx950: preprocessing.
//
// Method: FR summary ("Résumé Technique : Réduire le goulot d'étranglement de
// la mémoire GPU par la compression sans perte pour le ML") and KO summary
// ("Reducing the GPU Memory Bottleneck with Lossless Compression for ML --
// Extended"), section "Algorithme central" / "핵심 알고리즘", step 1: a batch
// of tensors is scanned for bit positions that hold the same value in at
// least a fraction T of them; the result is a fixed-size Mask and Bitval,
// kept in GPU memory and reused for the whole dataset.  Also the derived
// tables the encode and decode kernels read.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>
#include <stdint.h>

#include "ibp_device.hpp"
#include "ibp_internal.hpp"

namespace ibp {

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

static const uint32_t kPlanWpb[] = {4u, 8u, 12u, 16u};

// The launch shape depends only on the kernel, its LDS needs and the device,
// so it is worked out once per combination and kept (small launches would
// otherwise pay for the attribute queries on every call).
struct PlanKey {
    const void* kernel;
    size_t head, wave;
    uint32_t cu_count;
    uint32_t max_per_simd;
    int device;
    bool operator==(const PlanKey& o) const {
        return kernel == o.kernel && head == o.head && wave == o.wave && cu_count == o.cu_count &&
               max_per_simd == o.max_per_simd && device == o.device;
    }
};
struct PlanKeyHash {
    size_t operator()(const PlanKey& k) const {
        size_t h = std::hash<const void*>()(k.kernel);
        h = h * 1000003u ^ std::hash<size_t>()(k.head);
        h = h * 1000003u ^ std::hash<size_t>()(k.wave);
        return h * 1000003u ^ (size_t)k.cu_count ^ ((size_t)k.max_per_simd << 12) ^ ((size_t)k.device << 20);
    }
};

static bool plan_uncached(const void* kernel, size_t head_bytes, size_t wave_bytes, uint32_t cu_count,
                          uint32_t max_per_simd, PersistentPlan* plan) {
    hipFuncAttributes attr;
    uint32_t vgprs = 64, max_threads = 256;
    if (hipFuncGetAttributes(&attr, kernel) == hipSuccess) {
        if (attr.numRegs > 0) vgprs = (uint32_t)attr.numRegs;
        if (attr.maxThreadsPerBlock > 0) max_threads = (uint32_t)attr.maxThreadsPerBlock;
    }
    (void)hipGetLastError();
    int dev = 0, max_block_lds = 65536;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&max_block_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    (void)hipGetLastError();
    const uint64_t block_cap = max_block_lds > 0 ? (uint64_t)max_block_lds : 65536;
    // 512 VGPRs per SIMD lane, at most 8 waves per SIMD, 4 SIMDs per CU
    uint32_t per_simd = 512 / ((vgprs + 7) & ~7u);
    if (per_simd > 8) per_simd = 8;
    if (per_simd > max_per_simd) per_simd = max_per_simd;
    if (per_simd < 1) per_simd = 1;
    const uint32_t cu_waves = 4 * per_simd;
    PersistentPlan best;
    uint32_t best_waves = 0;
    // Waves per workgroup: the candidates the kernel's launch bounds allow,
    // keeping the one with the most resident waves (ties: the smaller
    // workgroup).  Larger groups share one LDS copy of the tables.
    for (uint32_t wpb : kPlanWpb) {
        if (wpb * kWave > max_threads) continue;
        const uint64_t shm = ((head_bytes + 15) & ~(size_t)15) + (uint64_t)wpb * wave_bytes;
        if (shm > block_cap || shm > kLdsPerCu) continue;
        uint64_t wgs = shm ? kLdsPerCu / shm : 64;
        if (wgs * wpb > cu_waves) wgs = cu_waves / wpb;
        if (wgs == 0) continue;
        const uint32_t waves = (uint32_t)(wgs * wpb);
        if (waves > best_waves) {
            best_waves = waves;
            best.wpb = wpb;
            best.shm = (size_t)shm;
            best.blocks = (uint32_t)(wgs * cu_count);
        }
    }
    if (!best_waves) return false;
    if (best.shm > 65536) {
        if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)best.shm) != hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
    }
    *plan = best;
    return true;
}

bool plan_persistent(const void* kernel, size_t head_bytes, size_t wave_bytes, uint32_t cu_count,
                     uint64_t n_items, PersistentPlan* plan, uint32_t max_waves_per_simd, uint64_t max_items) {
    static std::mutex mu;
    static std::unordered_map<PlanKey, std::pair<bool, PersistentPlan>, PlanKeyHash> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const PlanKey key{kernel, head_bytes, wave_bytes, cu_count, max_waves_per_simd, dev};
    std::pair<bool, PersistentPlan> entry;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end()) {
            entry = it->second;
        } else {
            entry.first = plan_uncached(kernel, head_bytes, wave_bytes, cu_count, max_waves_per_simd, &entry.second);
            cache.emplace(key, entry);
        }
    }
    if (!entry.first) return false;
    PersistentPlan p = entry.second;
    // Beyond max_items items per resident wave the launch adds workgroups
    // past the resident fill; the hardware dispatches them as earlier ones
    // retire, and each re-stages the tables once.
    if (max_items == 0) max_items = 1;
    const uint64_t want = (n_items + p.wpb - 1) / p.wpb;
    const uint64_t cap = (n_items + (uint64_t)p.wpb * max_items - 1) / ((uint64_t)p.wpb * max_items);
    uint64_t blocks = cap > p.blocks ? cap : (uint64_t)p.blocks;
    if (blocks > want) blocks = want;
    if (blocks > 0x7fffffffull) blocks = 0x7fffffffull;
    p.blocks = (uint32_t)blocks;
    *plan = p;
    return true;
}

}  // namespace ibp
