// ibp_api.hip -- host side of libibp: argument checks, the metadata handle,
// per-stream look-back scratch, and kernel dispatch.  The C ABI is declared
// in include/ibp.h; every step of the codec runs in the kernels of
// ibp_meta.hip, ibp_encode.hip and ibp_decode.hip.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/ibp.h"
#include "ibp_internal.hpp"

using namespace ibp;

namespace {

constexpr uint32_t kMaxPeriodBits = 1u << 20;
constexpr uint64_t kLineWords = 64;     // 256-byte first-read granule
constexpr uint64_t kMemLineWords = 32;  // 128-byte line that memory reads move

// Look-back scratch of one (handle, stream) pair.  The ticket counter is
// zeroed on the stream before every launch; only the epoch, which keeps a
// launch's status words apart from those of earlier launches, is counted on
// the host.
struct Scratch {
    unsigned long long* status = nullptr;
    uint64_t status_cap = 0;
    uint64_t* totals = nullptr;
    uint64_t totals_cap = 0;
    uint32_t* ticket = nullptr;
    uint32_t epoch = 0;
};

}  // namespace

struct ibp_meta_s {
    int device = 0;
    uint32_t cu_count = 0;
    uint64_t first_read_bytes = 0;  // 0: default policy
    uint64_t typical_item_bytes = 0; // median stored bytes over the metadata sample (0: unknown)
    ibp_params params{};
    uint32_t Mw = 0, Pc = 0, g = 0, log2g = 0, G = 0, Ne = 0;
    std::vector<uint32_t> mask_h, bitval_h;
    void* dmem = nullptr;
    uint32_t* d_mask = nullptr;
    uint32_t* d_bitval = nullptr;
    Summary* d_summary = nullptr;
    uint32_t* d_err = nullptr;
    Tables tabs{};
    Summary sum{};
    std::mutex mu;
    std::map<hipStream_t, Scratch> scratch;
};

namespace {

struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) {
            ok = false;
            return;
        }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

uint32_t gcd32(uint32_t a, uint32_t b) {
    while (b) {
        uint32_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

uint32_t bit_length(uint32_t v) {
    uint32_t n = 0;
    while (v) {
        ++n;
        v >>= 1;
    }
    return n;
}

ibp_status check_params(const ibp_params* p, bool need_threshold) {
    if (!p) return IBP_ERR_INVALID_ARG;
    const uint64_t L = p->tensor_bytes;
    const uint64_t W = p->chunk_bits, M = p->period_bits;
    if (L == 0 || L % 4 != 0 || W == 0 || M == 0) return IBP_ERR_INVALID_ARG;
    if ((8 * L) % W != 0 || M % W != 0 || (8 * L) % M != 0) return IBP_ERR_INVALID_ARG;
    if (need_threshold && !(p->threshold > 0.5 && p->threshold <= 1.0)) return IBP_ERR_INVALID_ARG;
    if (W < 32 || W > 1024 || (W & (W - 1)) != 0) return IBP_ERR_UNSUPPORTED;
    if (M > kMaxPeriodBits) return IBP_ERR_UNSUPPORTED;
    return IBP_OK;
}

enum class Kind { Device, Host, Bad };

Kind pointer_kind(const void* ptr, int device) {
    if (!ptr) return Kind::Bad;
    hipPointerAttribute_t a;
    memset(&a, 0, sizeof(a));
    if (hipPointerGetAttributes(&a, ptr) != hipSuccess) {
        (void)hipGetLastError();
        return Kind::Bad;
    }
    switch (a.type) {
        case hipMemoryTypeDevice:
            return a.device == device ? Kind::Device : Kind::Bad;
        case hipMemoryTypeManaged:
            return Kind::Device;
        case hipMemoryTypeHost:
            return Kind::Host;
        default:
            return Kind::Bad;
    }
}

bool device_or_pinned(const void* p, int dev) { return pointer_kind(p, dev) != Kind::Bad; }
bool device_only(const void* p, int dev) { return pointer_kind(p, dev) == Kind::Device; }

ibp_status from_hip(hipError_t e) {
    if (e == hipSuccess) return IBP_OK;
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? IBP_ERR_NOMEM : IBP_ERR_DEVICE;
}

#define IBP_TRY(expr)                        \
    do {                                     \
        ibp_status st_ = from_hip(expr);     \
        if (st_ != IBP_OK) return st_;       \
    } while (0)

// Allocates the handle's device tables and fills in its shape fields.
ibp_status new_handle(const ibp_params* p, ibp_meta_s** out) {
    ibp_meta_s* h = new (std::nothrow) ibp_meta_s();
    if (!h) return IBP_ERR_NOMEM;
    int cus = 0;
    if (hipGetDevice(&h->device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess) {
        (void)hipGetLastError();
        delete h;
        return IBP_ERR_DEVICE;
    }
    h->cu_count = cus > 0 ? (uint32_t)cus : 1u;
    h->params = *p;
    h->Mw = p->period_bits / 32;
    h->Pc = p->period_bits / p->chunk_bits;
    h->g = p->chunk_bits / 32;
    h->log2g = bit_length(h->g) - 1;
    h->G = gcd32(32, h->Pc);
    h->Ne = h->Pc / h->G;
    const uint64_t Mw = h->Mw;
    // layout (words): mask, bitval, kd, dx[4], r[16], planes[Ne*11], summary, err
    const uint64_t words = Mw * (3 + 4 + kMaxRuns) + (uint64_t)h->Ne * kPlanes;
    const uint64_t bytes = words * 4 + 256 + sizeof(Summary) + 64;
    hipError_t e = hipMalloc(&h->dmem, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        delete h;
        return IBP_ERR_NOMEM;
    }
    uint32_t* w = static_cast<uint32_t*>(h->dmem);
    h->d_mask = w;
    h->d_bitval = w + Mw;
    uint32_t* kd = w + 2 * Mw;
    uint32_t* dx = w + 3 * Mw;
    uint32_t* r = w + 7 * Mw;
    uint32_t* planes = w + (7 + kMaxRuns) * Mw;
    uintptr_t tail = reinterpret_cast<uintptr_t>(planes + (uint64_t)h->Ne * kPlanes);
    tail = (tail + 255) & ~uintptr_t(255);
    h->d_summary = reinterpret_cast<Summary*>(tail);
    h->d_err = reinterpret_cast<uint32_t*>(tail + ((sizeof(Summary) + 63) & ~size_t(63)));
    h->tabs = Tables{h->d_mask, h->d_bitval, kd, dx, r, planes};
    *out = h;
    return IBP_OK;
}

// Derived tables from the device Mask/Bitval, then the host copies.
ibp_status finish_handle(ibp_meta_s* h, hipStream_t s) {
    Summary init{};
    init.uniform = 1;
    IBP_TRY(hipMemcpyAsync(h->d_summary, &init, sizeof(init), hipMemcpyHostToDevice, s));
    IBP_TRY(launch_fill_u32(h->d_err, 1, 0, s));
    uint32_t* kd = const_cast<uint32_t*>(h->tabs.kd);
    uint32_t* dx = const_cast<uint32_t*>(h->tabs.dx);
    uint32_t* r = const_cast<uint32_t*>(h->tabs.r);
    uint32_t* pl = const_cast<uint32_t*>(h->tabs.planes);
    IBP_TRY(launch_tables(h->d_mask, h->d_bitval, h->Mw, h->Pc, h->g, h->G, kd, dx, r, pl, h->d_summary, s));
    h->mask_h.resize(h->Mw);
    h->bitval_h.resize(h->Mw);
    IBP_TRY(hipMemcpyAsync(h->mask_h.data(), h->d_mask, 4ull * h->Mw, hipMemcpyDeviceToHost, s));
    IBP_TRY(hipMemcpyAsync(h->bitval_h.data(), h->d_bitval, 4ull * h->Mw, hipMemcpyDeviceToHost, s));
    IBP_TRY(hipMemcpyAsync(&h->sum, h->d_summary, sizeof(Summary), hipMemcpyDeviceToHost, s));
    IBP_TRY(hipStreamSynchronize(s));
    return IBP_OK;
}

// Median stored bytes (record, or L when raw) over the metadata sample, from
// the record-length kernel; sets typical_item_bytes, or leaves it 0 when the
// geometry has no record-length kernel.  Synchronous (the handle is being
// built).
ibp_status sample_item_stats(ibp_meta_s* h, const void* sample, uint64_t n_sample, hipStream_t s);

void free_handle(ibp_meta_s* h) {
    if (!h) return;
    (void)hipDeviceSynchronize();
    for (auto& kv : h->scratch) {
        if (kv.second.status) (void)hipFree(kv.second.status);
        if (kv.second.totals) (void)hipFree(kv.second.totals);
        if (kv.second.ticket) (void)hipFree(kv.second.ticket);
    }
    if (h->dmem) (void)hipFree(h->dmem);
    delete h;
}

uint64_t min_record_bits(const ibp_meta_s* h) {
    const uint64_t L = h->params.tensor_bytes;
    const uint64_t n_chunks = 8 * L / h->params.chunk_bits;
    const uint64_t H = 32 * ((n_chunks + 31) / 32);
    const uint64_t periods = 8 * L / h->params.period_bits;
    return H + 8 * L - periods * h->sum.invariant_bits;
}

Geo make_geo(const ibp_meta_s* h, bool aligned16, uint32_t long_tile_words) {
    Geo g{};
    const uint64_t L = h->params.tensor_bytes;
    g.L = L;
    g.n_words = L / 4;
    g.n_chunks = 8 * L / h->params.chunk_bits;
    g.hdr_words = (g.n_chunks + 31) / 32;
    g.Mw = h->Mw;
    g.Pc = h->Pc;
    g.log2g = h->log2g;
    g.G = h->G;
    g.np = bit_length(h->sum.max_chunk_k);
    if (g.np > (uint32_t)kPlanes) g.np = kPlanes;
    g.k1 = g.Pc == 1 ? h->sum.max_chunk_k : 0;
    g.aligned16 = aligned16 ? 1u : 0u;
    if (g.n_words <= kMaxTileWords) {
        g.tile_words = (uint32_t)g.n_words;
        g.tiles_per_tensor = 1;
    } else {
        g.tile_words = long_tile_words;
        g.tiles_per_tensor = (g.n_words + long_tile_words - 1) / long_tile_words;
    }
    // First read of a single-tile record: every record is at least min_words
    // long, so the read is cut at the last 256-byte boundary inside that
    // prefix, and is never shorter than 256 bytes (the second read then starts
    // on a 256-byte boundary; zero-copy reads of pinned host memory measured
    // fastest with this split).  Memory moves whole 128-byte lines, so when
    // the shortest record already covers all but 1/16 of the slot's lines,
    // the whole slot is read at once instead of paying a second round trip.
    const uint64_t min_words = (min_record_bits(h) + 31) / 32;
    const uint64_t slot_lines = (g.n_words + kMemLineWords - 1) / kMemLineWords;
    const uint64_t min_lines = (min_words + kMemLineWords - 1) / kMemLineWords;
    uint64_t spec;
    if (h->first_read_bytes) {
        spec = (h->first_read_bytes + 3) / 4;
        if (spec < g.hdr_words) spec = g.hdr_words;
    } else if (min_lines >= slot_lines || (slot_lines - min_lines) * 16 <= slot_lines) {
        spec = g.n_words;
    } else {
        spec = (min_words / kLineWords) * kLineWords;
        if (spec < kLineWords) spec = kLineWords;
        // records of the sample mostly shorter than that: one 128-byte line
        // (rounded up to whole lines) covers the usual record in one read
        if (h->typical_item_bytes) {
            const uint64_t usual = (h->typical_item_bytes + 4 * kMemLineWords - 1) / (4 * kMemLineWords) * kMemLineWords;
            if (usual < spec) spec = usual;
        }
        if (spec < g.hdr_words) spec = g.hdr_words;
    }
    if (aligned16) spec = (spec + 3) & ~3ull;
    if (spec > g.n_words) spec = g.n_words;
    g.spec_words = (uint32_t)spec;
    return g;
}

bool aligned16(uint64_t L, std::initializer_list<const void*> ptrs) {
    if (L % 16 != 0) return false;
    for (const void* p : ptrs)
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return false;
    return true;
}

ibp_status sample_item_stats(ibp_meta_s* h, const void* sample, uint64_t n_sample, hipStream_t s) {
    const uint64_t L = h->params.tensor_bytes;
    const Geo geo = make_geo(h, aligned16(L, {sample}), kLongTileWordsEncode);
    if (!packed_supported(geo, h->sum.max_runs, h->sum.uniform != 0)) return IBP_OK;
    uint64_t* d_sizes = nullptr;
    IBP_TRY(hipMalloc(&d_sizes, n_sample * sizeof(uint64_t)));
    std::vector<uint64_t> sizes(n_sample);
    hipError_t e = launch_item_sizes(h->tabs, geo, h->sum.max_runs, h->sum.uniform != 0, sample, n_sample, d_sizes,
                                     h->cu_count, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(sizes.data(), d_sizes, n_sample * sizeof(uint64_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    (void)hipFree(d_sizes);
    IBP_TRY(e);
    std::nth_element(sizes.begin(), sizes.begin() + n_sample / 2, sizes.end());
    h->typical_item_bytes = sizes[n_sample / 2];
    return IBP_OK;
}

// IBP_ERR_UNSUPPORTED while `s` is capturing a graph: a look-back launch
// refers to its stream's scratch and epoch at the time of the call, which a
// replay would not renew.
ibp_status refuse_capture(hipStream_t s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return IBP_ERR_DEVICE;
    }
    return cs == hipStreamCaptureStatusNone ? IBP_OK : IBP_ERR_UNSUPPORTED;
}

// Look-back state for one launch with `tiles` status words (one per tile of
// the multi-tile encode, per group of tiles of the decode, per block of the
// offsets scan) on stream s: grows the per-stream buffers when needed and
// queues the zeroing of the ticket counter on s.  Returns with `lock` holding the handle's mutex; the caller
// queues its launch before releasing it, so launches on one stream from
// several host threads reach the stream in the order of their reservations
// and no buffer is replaced while a reserved launch is still to be queued.
ibp_status lookback_for(ibp_meta_s* h, hipStream_t s, uint64_t tiles, uint64_t tensors, LookBack* lb,
                        std::unique_lock<std::mutex>* lock) {
    ibp_status st = refuse_capture(s);
    if (st != IBP_OK) return st;
    *lock = std::unique_lock<std::mutex>(h->mu);
    Scratch& sc = h->scratch[s];
    if (!sc.ticket) IBP_TRY(hipMalloc(&sc.ticket, 256));
    if (sc.status_cap < tiles) {
        // earlier launches on s were queued under the mutex: once s is idle
        // nothing refers to the old buffer
        IBP_TRY(hipStreamSynchronize(s));
        if (sc.status) IBP_TRY(hipFree(sc.status));
        sc.status = nullptr;
        sc.status_cap = 0;
        IBP_TRY(hipMalloc(&sc.status, tiles * sizeof(unsigned long long)));
        IBP_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(sc.status), 2 * tiles, 0, s));
        sc.status_cap = tiles;
        sc.epoch = 0;
    }
    if (sc.totals_cap < tensors) {
        IBP_TRY(hipStreamSynchronize(s));
        if (sc.totals) IBP_TRY(hipFree(sc.totals));
        sc.totals = nullptr;
        sc.totals_cap = 0;
        IBP_TRY(hipMalloc(&sc.totals, tensors * sizeof(uint64_t)));
        sc.totals_cap = tensors;
    }
    sc.epoch += 1;
    if (sc.epoch >= (1u << 20)) {
        IBP_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(sc.status), 2 * sc.status_cap, 0, s));
        sc.epoch = 1;
    }
    IBP_TRY(launch_fill_u32(sc.ticket, 1, 0, s));
    lb->status = sc.status;
    lb->ticket = sc.ticket;
    lb->epoch = sc.epoch;
    lb->totals = sc.totals;
    lb->err = h->d_err;
    return IBP_OK;
}

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

const char* ibp_status_string(ibp_status s) {
    switch (s) {
        case IBP_OK: return "ok";
        case IBP_ERR_INVALID_ARG: return "invalid argument";
        case IBP_ERR_UNSUPPORTED: return "unsupported format";
        case IBP_ERR_DEVICE: return "HIP error";
        case IBP_ERR_NOMEM: return "out of memory";
        case IBP_ERR_CORRUPT: return "corrupt record";
        case IBP_ERR_RANGE: return "id out of range";
        case IBP_ERR_TOO_LARGE: return "more tiles than the static scratch of ibp_decompress_noalloc holds";
    }
    return "unknown status";
}

ibp_status ibp_build_metadata(const ibp_params* params, const void* sample, uint64_t n_sample,
                              ibp_meta_t* out, hipStream_t stream) {
    if (!out) return IBP_ERR_INVALID_ARG;
    ibp_status st = check_params(params, true);
    if (st != IBP_OK) return st;
    int dev = 0;
    IBP_TRY(hipGetDevice(&dev));
    if (n_sample == 0 || !device_or_pinned(sample, dev)) return IBP_ERR_INVALID_ARG;
    const uint64_t L = params->tensor_bytes;
    const uint64_t per = 8 * L / params->period_bits;
    if (n_sample > (1ull << 40) / per) return IBP_ERR_INVALID_ARG;
    const uint64_t n_obs = n_sample * per;
    if (n_obs >= (1ull << 32)) return IBP_ERR_INVALID_ARG;
    // K = ceil(T * n_obs), product rounded to nearest in IEEE double.
    const double prod = params->threshold * (double)n_obs;
    const uint64_t K = (uint64_t)ceil(prod);

    ibp_meta_s* h = nullptr;
    st = new_handle(params, &h);
    if (st != IBP_OK) return st;
    uint32_t* counts = nullptr;
    hipError_t e = hipMalloc(&counts, 4ull * params->period_bits);
    if (e == hipSuccess) e = launch_fill_u32(counts, params->period_bits, 0, stream);
    if (e == hipSuccess)
        e = launch_meta_hist(static_cast<const uint32_t*>(sample), n_sample * (L / 4), h->Mw, counts, stream);
    if (e == hipSuccess) e = launch_meta_finalize(counts, h->Mw, n_obs, K, h->d_mask, h->d_bitval, stream);
    st = from_hip(e);
    if (st == IBP_OK) st = finish_handle(h, stream);
    if (st == IBP_OK) st = sample_item_stats(h, sample, n_sample, stream);
    if (counts) (void)hipFree(counts);
    if (st != IBP_OK) {
        free_handle(h);
        return st;
    }
    *out = h;
    return IBP_OK;
}

ibp_status ibp_meta_create(const ibp_params* params, const uint32_t* mask, const uint32_t* bitval,
                           ibp_meta_t* out, hipStream_t stream) {
    if (!out || !mask || !bitval) return IBP_ERR_INVALID_ARG;
    ibp_status st = check_params(params, false);
    if (st != IBP_OK) return st;
    const uint32_t Mw = params->period_bits / 32;
    for (uint32_t i = 0; i < Mw; ++i)
        if (bitval[i] & ~mask[i]) return IBP_ERR_INVALID_ARG;
    ibp_meta_s* h = nullptr;
    st = new_handle(params, &h);
    if (st != IBP_OK) return st;
    hipError_t e = hipMemcpyAsync(h->d_mask, mask, 4ull * Mw, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(h->d_bitval, bitval, 4ull * Mw, hipMemcpyHostToDevice, stream);
    st = from_hip(e);
    if (st == IBP_OK) st = finish_handle(h, stream);
    if (st != IBP_OK) {
        free_handle(h);
        return st;
    }
    *out = h;
    return IBP_OK;
}

ibp_status ibp_meta_get(ibp_meta_t h, ibp_params* params, uint32_t* mask, uint32_t* bitval) {
    if (!h) return IBP_ERR_INVALID_ARG;
    if (params) *params = h->params;
    if (mask) memcpy(mask, h->mask_h.data(), 4ull * h->Mw);
    if (bitval) memcpy(bitval, h->bitval_h.data(), 4ull * h->Mw);
    return IBP_OK;
}

ibp_status ibp_meta_get_info(ibp_meta_t h, ibp_meta_info* info) {
    if (!h || !info) return IBP_ERR_INVALID_ARG;
    info->invariant_bits = h->sum.invariant_bits;
    info->min_record_bytes = 4 * ((min_record_bits(h) + 31) / 32);
    info->max_runs = h->sum.max_runs;
    info->uniform = h->sum.uniform;
    return IBP_OK;
}

ibp_status ibp_meta_set_first_read(ibp_meta_t h, uint64_t bytes) {
    if (!h) return IBP_ERR_INVALID_ARG;
    h->first_read_bytes = bytes;
    return IBP_OK;
}

ibp_status ibp_meta_destroy(ibp_meta_t h) {
    if (!h) return IBP_ERR_INVALID_ARG;
    DeviceGuard guard(h->device);
    free_handle(h);
    return IBP_OK;
}

ibp_status ibp_compress(ibp_meta_t h, const void* src, uint64_t n_tensors, void* dst_slots,
                        uint32_t* bitmask, uint64_t* stored_bytes, hipStream_t stream) {
    if (!h) return IBP_ERR_INVALID_ARG;
    if (n_tensors == 0) return IBP_OK;
    DeviceGuard guard(h->device);
    if (!guard.ok) return IBP_ERR_DEVICE;
    const uint64_t L = h->params.tensor_bytes;
    if (n_tensors > (~0ull) / L) return IBP_ERR_INVALID_ARG;
    if (!device_or_pinned(src, h->device) || !device_or_pinned(dst_slots, h->device)) return IBP_ERR_INVALID_ARG;
    if (!device_only(bitmask, h->device)) return IBP_ERR_INVALID_ARG;
    if (stored_bytes && !device_only(stored_bytes, h->device)) return IBP_ERR_INVALID_ARG;
    if (overlaps(src, n_tensors * L, dst_slots, n_tensors * L)) return IBP_ERR_INVALID_ARG;
    Geo geo = make_geo(h, aligned16(L, {src, dst_slots}), kLongTileWordsEncode);
    geo.src_in_hbm = pointer_kind(src, h->device) == Kind::Device;
    geo.dst_in_hbm = pointer_kind(dst_slots, h->device) == Kind::Device;
    LookBack lb{};
    std::unique_lock<std::mutex> lock;
    if (geo.tiles_per_tensor > 1) {
        ibp_status st = lookback_for(h, stream, encode_status_words(geo, n_tensors), n_tensors, &lb, &lock);
        if (st != IBP_OK) return st;
    }
    return from_hip(launch_encode(h->tabs, geo, h->sum.max_runs, h->sum.uniform != 0, src, n_tensors, dst_slots,
                                  bitmask, stored_bytes, &lb, h->cu_count, stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Static look-back scratch of ibp_decompress_noalloc: one array per GPU,
// loaded with the library's code object and kept until the process ends.
// Words [0, 32) hold the ticket counter, the status words of the tiles
// follow.  Host code never passes the array's name to a kernel or a copy:
// its device address comes from hipGetSymbolAddress, once per device.
// ---------------------------------------------------------------------------
namespace {
constexpr uint64_t kNoAllocScratchWords = IBP_NOALLOC_SCRATCH_BYTES / 8;
constexpr uint64_t kNoAllocHeadWords = 32;
constexpr int kMaxDevices = 64;
static_assert(IBP_NOALLOC_MAX_TILES == kNoAllocScratchWords - kNoAllocHeadWords, "scratch layout");
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) unsigned long long scratch[kNoAllocScratchWords];

// Device address of `scratch` on `dev` (the current device), looked up on
// the first use on that device.
static ibp_status noalloc_scratch(int dev, unsigned long long** out) {
    if (dev < 0 || dev >= kMaxDevices) return IBP_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return IBP_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<unsigned long long*>(g_scratch_ptr[dev]);
    return IBP_OK;
}

// Look-back state of one launch with `entries` status words (one per group of
// tiles) in the static scratch: the ticket and the status words are zeroed
// by fill kernels on the stream (no memset node, so the call may be captured
// in a graph), and the epoch is always 1.
static ibp_status noalloc_lookback(ibp_meta_s* h, hipStream_t s, uint64_t entries, LookBack* lb) {
    unsigned long long* base = nullptr;
    ibp_status st = noalloc_scratch(h->device, &base);
    if (st != IBP_OK) return st;
    uint32_t* ticket = reinterpret_cast<uint32_t*>(base);
    unsigned long long* status = base + kNoAllocHeadWords;
    IBP_TRY(launch_fill_u32(ticket, 1, 0, s));
    IBP_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(status), 2 * entries, 0, s));
    lb->status = status;
    lb->ticket = ticket;
    lb->epoch = 1;
    lb->totals = nullptr;
    lb->err = h->d_err;
    return IBP_OK;
}

extern "C" {

static ibp_status decode_common(ibp_meta_t h, const void* slots, uint64_t n_slots, const uint32_t* bitmask,
                                const int64_t* ids, uint64_t n_out, void* dst, hipStream_t stream,
                                bool static_scratch = false) {
    if (!h) return IBP_ERR_INVALID_ARG;
    if (n_out == 0) return IBP_OK;
    const uint64_t L = h->params.tensor_bytes;
    // the static scratch holds one status word per group, and a group spans
    // at least one 2,048-word tile's worth of words on either path
    static_assert(kDecodeTilesPerGroupHbm * kLongTileWordsDecodeHbm >= kLongTileWordsDecode &&
                      kDecodeTilesPerGroup >= 1,
                  "groups per tensor must not exceed its 2,048-word tiles");
    if (static_scratch && L / 4 > kMaxTileWords) {
        const uint64_t tpt = (L / 4 + kLongTileWordsDecode - 1) / kLongTileWordsDecode;
        if (n_out > IBP_NOALLOC_MAX_TILES / tpt) return IBP_ERR_TOO_LARGE;
    }
    DeviceGuard guard(h->device);
    if (!guard.ok) return IBP_ERR_DEVICE;
    if (n_out > (~0ull) / L || n_slots > (~0ull) / L) return IBP_ERR_INVALID_ARG;
    const Kind slots_kind = pointer_kind(slots, h->device);
    if (slots_kind == Kind::Bad) return IBP_ERR_INVALID_ARG;
    if (!device_only(bitmask, h->device) || !device_only(dst, h->device)) return IBP_ERR_INVALID_ARG;
    if (ids && !device_only(ids, h->device)) return IBP_ERR_INVALID_ARG;
    if (overlaps(slots, n_slots * L, dst, n_out * L)) return IBP_ERR_INVALID_ARG;
    Geo geo = make_geo(h, aligned16(L, {slots, dst}), decode_tile_words(slots_kind == Kind::Device));
    geo.src_in_hbm = slots_kind == Kind::Device;
    LookBack lb{};
    std::unique_lock<std::mutex> lock;
    if (geo.tiles_per_tensor > 1) {
        // one status word per group of tiles (look-back entries, or the
        // group start bits when the records are in HBM)
        const uint64_t groups = n_out * tile_groups(geo.tiles_per_tensor, decode_group_tiles(geo.src_in_hbm));
        ibp_status st = static_scratch ? noalloc_lookback(h, stream, groups, &lb)
                                       : lookback_for(h, stream, groups, 0, &lb, &lock);
        if (st != IBP_OK) return st;
    }
    return from_hip(launch_decode(h->tabs, geo, h->sum.max_runs, h->sum.uniform != 0, slots, n_slots, bitmask,
                                  ids, n_out, dst, h->d_err, &lb, h->cu_count, stream));
}

ibp_status ibp_decompress(ibp_meta_t h, const void* slots, const uint32_t* bitmask, uint64_t n_tensors,
                          void* dst, hipStream_t stream) {
    return decode_common(h, slots, n_tensors, bitmask, nullptr, n_tensors, dst, stream);
}

ibp_status ibp_decompress_noalloc(ibp_meta_t h, const void* slots, const uint32_t* bitmask, uint64_t n_tensors,
                                  void* dst, hipStream_t stream) {
    return decode_common(h, slots, n_tensors, bitmask, nullptr, n_tensors, dst, stream, true);
}

ibp_status ibp_gather_decompress(ibp_meta_t h, const void* slots, uint64_t n_slots, const uint32_t* bitmask,
                                 const int64_t* ids, uint64_t n_ids, void* dst, hipStream_t stream) {
    if (n_ids && !ids) return IBP_ERR_INVALID_ARG;
    return decode_common(h, slots, n_slots, bitmask, ids, n_ids, dst, stream);
}

// ---------------------------------------------------------------------------
// Packed cache.
// ---------------------------------------------------------------------------
ibp_status ibp_packed_offsets(ibp_meta_t h, const void* src, uint64_t n_tensors, uint64_t* offsets,
                              hipStream_t stream) {
    if (!h || !offsets) return IBP_ERR_INVALID_ARG;
    DeviceGuard guard(h->device);
    if (!guard.ok) return IBP_ERR_DEVICE;
    const uint64_t L = h->params.tensor_bytes;
    if (n_tensors > (~0ull) / L - 1) return IBP_ERR_INVALID_ARG;
    if (!device_only(offsets, h->device) || reinterpret_cast<uintptr_t>(offsets) % 8) return IBP_ERR_INVALID_ARG;
    if (n_tensors && !device_or_pinned(src, h->device)) return IBP_ERR_INVALID_ARG;
    const Geo geo = make_geo(h, aligned16(L, {src}), kLongTileWordsEncode);
    const bool uni = h->sum.uniform != 0;
    if (!packed_supported(geo, h->sum.max_runs, uni) || !packed_decode_supported(geo, h->sum.max_runs, uni))
        return IBP_ERR_UNSUPPORTED;
    if (n_tensors) {
        // the offsets scan below takes look-back scratch: refused under
        // capture before anything is queued
        ibp_status st = refuse_capture(stream);
        if (st != IBP_OK) return st;
        IBP_TRY(launch_item_sizes(h->tabs, geo, h->sum.max_runs, uni, src, n_tensors, offsets + 1, h->cu_count,
                                  stream));
    }
    LookBack lb{};
    std::unique_lock<std::mutex> lock;
    const uint64_t blocks = (n_tensors + kScanBlock - 1) / kScanBlock;
    if (n_tensors) {
        ibp_status st = lookback_for(h, stream, blocks, 0, &lb, &lock);
        if (st != IBP_OK) return st;
    }
    return from_hip(launch_scan_sizes(offsets, n_tensors, lb, stream));
}

ibp_status ibp_compress_packed(ibp_meta_t h, const void* src, uint64_t n_tensors, const uint64_t* offsets,
                               void* dst, uint64_t capacity, uint32_t* bitmask, hipStream_t stream) {
    if (!h || !offsets) return IBP_ERR_INVALID_ARG;
    if (n_tensors == 0) return IBP_OK;
    DeviceGuard guard(h->device);
    if (!guard.ok) return IBP_ERR_DEVICE;
    const uint64_t L = h->params.tensor_bytes;
    if (n_tensors > (~0ull) / L - 1) return IBP_ERR_INVALID_ARG;
    if (!device_or_pinned(src, h->device) || !device_or_pinned(dst, h->device)) return IBP_ERR_INVALID_ARG;
    if (!device_only(offsets, h->device) || !device_only(bitmask, h->device)) return IBP_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(offsets) % 8) return IBP_ERR_INVALID_ARG;
    if (overlaps(src, n_tensors * L, dst, capacity)) return IBP_ERR_INVALID_ARG;
    const Geo geo = make_geo(h, aligned16(L, {src, dst}), kLongTileWordsEncode);
    const bool uni = h->sum.uniform != 0;
    if (!packed_supported(geo, h->sum.max_runs, uni)) return IBP_ERR_UNSUPPORTED;
    return from_hip(launch_encode_packed(h->tabs, geo, h->sum.max_runs, uni, src, n_tensors, dst,
                                         Items{offsets, capacity}, bitmask, h->d_err, h->cu_count, stream));
}

static ibp_status decode_packed_common(ibp_meta_t h, const void* buf, uint64_t buf_bytes, const uint64_t* offsets,
                                       uint64_t n_items, const uint32_t* bitmask, const int64_t* ids,
                                       uint64_t n_out, void* dst, hipStream_t stream) {
    if (!h || !offsets) return IBP_ERR_INVALID_ARG;
    if (n_out == 0) return IBP_OK;
    DeviceGuard guard(h->device);
    if (!guard.ok) return IBP_ERR_DEVICE;
    const uint64_t L = h->params.tensor_bytes;
    if (n_out > (~0ull) / L) return IBP_ERR_INVALID_ARG;
    const Kind buf_kind = pointer_kind(buf, h->device);
    if (buf_kind == Kind::Bad) return IBP_ERR_INVALID_ARG;
    if (!device_only(offsets, h->device) || !device_only(bitmask, h->device) || !device_only(dst, h->device))
        return IBP_ERR_INVALID_ARG;
    if (ids && !device_only(ids, h->device)) return IBP_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(offsets) % 8) return IBP_ERR_INVALID_ARG;
    if (overlaps(buf, buf_bytes, dst, n_out * L)) return IBP_ERR_INVALID_ARG;
    Geo geo = make_geo(h, aligned16(L, {buf, dst}), kLongTileWordsDecode);
    geo.src_in_hbm = buf_kind == Kind::Device;
    const bool uni = h->sum.uniform != 0;
    if (!packed_decode_supported(geo, h->sum.max_runs, uni)) return IBP_ERR_UNSUPPORTED;
    // an item's length is known from the offsets: read it whole at once
    geo.spec_words = (uint32_t)geo.n_words;
    const Items items{offsets, buf_bytes};
    return from_hip(launch_decode(h->tabs, geo, h->sum.max_runs, uni, buf, n_items, bitmask, ids, n_out, dst,
                                  h->d_err, nullptr, h->cu_count, stream, &items));
}

ibp_status ibp_decompress_packed(ibp_meta_t h, const void* buf, uint64_t buf_bytes, const uint64_t* offsets,
                                 const uint32_t* bitmask, uint64_t n_items, void* dst, hipStream_t stream) {
    return decode_packed_common(h, buf, buf_bytes, offsets, n_items, bitmask, nullptr, n_items, dst, stream);
}

ibp_status ibp_gather_decompress_packed(ibp_meta_t h, const void* buf, uint64_t buf_bytes, const uint64_t* offsets,
                                        uint64_t n_items, const uint32_t* bitmask, const int64_t* ids,
                                        uint64_t n_ids, void* dst, hipStream_t stream) {
    if (n_ids && !ids) return IBP_ERR_INVALID_ARG;
    return decode_packed_common(h, buf, buf_bytes, offsets, n_items, bitmask, ids, n_ids, dst, stream);
}

// ---------------------------------------------------------------------------
// Headers in GPU memory.
// ---------------------------------------------------------------------------
ibp_status ibp_compress_split(ibp_meta_t h, const void* src, uint64_t n_tensors, void* dst_slots, uint32_t* headers,
                              uint32_t* bitmask, uint64_t* stored_bytes, hipStream_t stream) {
    if (!h) return IBP_ERR_INVALID_ARG;
    if (n_tensors == 0) return IBP_OK;
    DeviceGuard guard(h->device);
    if (!guard.ok) return IBP_ERR_DEVICE;
    const uint64_t L = h->params.tensor_bytes;
    if (n_tensors > (~0ull) / L) return IBP_ERR_INVALID_ARG;
    if (!device_or_pinned(src, h->device) || !device_or_pinned(dst_slots, h->device)) return IBP_ERR_INVALID_ARG;
    if (!device_only(bitmask, h->device) || !device_only(headers, h->device)) return IBP_ERR_INVALID_ARG;
    if (stored_bytes && !device_only(stored_bytes, h->device)) return IBP_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(headers) % 4) return IBP_ERR_INVALID_ARG;
    if (overlaps(src, n_tensors * L, dst_slots, n_tensors * L)) return IBP_ERR_INVALID_ARG;
    const Geo geo = make_geo(h, aligned16(L, {src, dst_slots}), kLongTileWordsEncode);
    if (!split_supported(geo, h->sum.max_runs, h->sum.uniform != 0)) return IBP_ERR_UNSUPPORTED;
    return from_hip(launch_encode_split(h->tabs, geo, h->sum.max_runs, h->sum.uniform != 0, src, n_tensors,
                                        dst_slots, headers, bitmask, stored_bytes, h->cu_count, stream));
}

static ibp_status decode_split_common(ibp_meta_t h, const void* slots, uint64_t n_slots, const uint32_t* headers,
                                      const uint32_t* bitmask, const int64_t* ids, uint64_t n_out, void* dst,
                                      hipStream_t stream) {
    if (!h) return IBP_ERR_INVALID_ARG;
    if (n_out == 0) return IBP_OK;
    DeviceGuard guard(h->device);
    if (!guard.ok) return IBP_ERR_DEVICE;
    const uint64_t L = h->params.tensor_bytes;
    if (n_out > (~0ull) / L || n_slots > (~0ull) / L) return IBP_ERR_INVALID_ARG;
    const Kind slots_kind = pointer_kind(slots, h->device);
    if (slots_kind == Kind::Bad) return IBP_ERR_INVALID_ARG;
    if (!device_only(bitmask, h->device) || !device_only(dst, h->device) || !device_only(headers, h->device))
        return IBP_ERR_INVALID_ARG;
    if (ids && !device_only(ids, h->device)) return IBP_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(headers) % 4) return IBP_ERR_INVALID_ARG;
    if (overlaps(slots, n_slots * L, dst, n_out * L)) return IBP_ERR_INVALID_ARG;
    Geo geo = make_geo(h, aligned16(L, {slots, dst}), kLongTileWordsDecode);
    geo.src_in_hbm = slots_kind == Kind::Device;
    const bool uni = h->sum.uniform != 0;
    if (geo.hdr_words > kMaxSplitHeaderWords || !packed_decode_supported(geo, h->sum.max_runs, uni))
        return IBP_ERR_UNSUPPORTED;
    return from_hip(launch_decode(h->tabs, geo, h->sum.max_runs, uni, slots, n_slots, bitmask, ids, n_out, dst,
                                  h->d_err, nullptr, h->cu_count, stream, nullptr, headers));
}

ibp_status ibp_decompress_split(ibp_meta_t h, const void* slots, const uint32_t* headers, const uint32_t* bitmask,
                                uint64_t n_tensors, void* dst, hipStream_t stream) {
    return decode_split_common(h, slots, n_tensors, headers, bitmask, nullptr, n_tensors, dst, stream);
}

ibp_status ibp_gather_decompress_split(ibp_meta_t h, const void* slots, uint64_t n_slots, const uint32_t* headers,
                                       const uint32_t* bitmask, const int64_t* ids, uint64_t n_ids, void* dst,
                                       hipStream_t stream) {
    if (n_ids && !ids) return IBP_ERR_INVALID_ARG;
    return decode_split_common(h, slots, n_slots, headers, bitmask, ids, n_ids, dst, stream);
}

ibp_status ibp_check(ibp_meta_t h, hipStream_t stream) {
    if (!h) return IBP_ERR_INVALID_ARG;
    DeviceGuard guard(h->device);
    IBP_TRY(hipStreamSynchronize(stream));
    uint32_t v = 0;
    IBP_TRY(hipMemcpy(&v, h->d_err, 4, hipMemcpyDeviceToHost));
    if (v == kErrNone) return IBP_OK;
    IBP_TRY(launch_fill_u32(h->d_err, 1, 0, stream));
    IBP_TRY(hipStreamSynchronize(stream));
    if (v == kErrRange) return IBP_ERR_RANGE;
    return v == kErrStall ? IBP_ERR_DEVICE : IBP_ERR_CORRUPT;
}

}  // extern "C"
