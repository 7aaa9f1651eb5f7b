// lrs_host.hip -- host driver and C ABI of the LSD radix sort (gfx950).
//
// A sort is: one clear of the workspace counters, one all-pass digit
// histogram, then one sweep launch per digit pass, low digit first, each
// reading the previous pass's output (CUDA Handbook ch.16: the driver runs one
// pass per digit, ping-ponging two buffers; here the caller's output is one of
// the two and the rotation is chosen so the last pass lands in it, so the
// input is never written).  Everything is enqueued on the caller's stream; the
// library allocates nothing.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/lsd_radix_sort.h"
#include "lrs_launch.h"

namespace lrs {

// --------------------------------------------------- utility kernels

// Zero `words` u32 words at each of up to three regions.
struct ClearArgs {
    uint32_t *p[3];
    uint64_t words[3];
};

__global__ __launch_bounds__(kBlock) void clear_kernel(ClearArgs a) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (int r = 0; r < 3; ++r) {
        uint32_t *p = a.p[r];
        if (p == nullptr) continue;
        const uint64_t n = a.words[r];
        const uint64_t n4 = n / 4;  // regions are 16-byte aligned
        uint4 *p4 = reinterpret_cast<uint4 *>(p);
        for (uint64_t i = blockIdx.x * static_cast<uint64_t>(kBlock) + threadIdx.x; i < n4; i += stride)
            p4[i] = make_uint4(0u, 0u, 0u, 0u);
        for (uint64_t i = n4 * 4 + blockIdx.x * static_cast<uint64_t>(kBlock) + threadIdx.x; i < n; i += stride)
            p[i] = 0u;
    }
}

// Plain streaming copy: one 16-byte word per thread and a grid that covers the
// buffer once (a grid-stride loop only past 2^20 workgroups).  On MI355X this
// shape moves about 6.1 TB/s; unrolled or grid-stride shapes with more bytes
// per thread in flight lose a quarter of that or more.
__global__ __launch_bounds__(kBlock) void copy_kernel(const uint4 *src, uint4 *dst, uint64_t n16,
                                                      const uint8_t *src_tail, uint8_t *dst_tail,
                                                      uint32_t tail) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = blockIdx.x * static_cast<uint64_t>(kBlock) + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
    if (blockIdx.x == 0 && threadIdx.x < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}


namespace {

#ifndef LRS_MIN_TILES
#define LRS_MIN_TILES 256
#endif
// Fewest tiles a larger tile shape must still give: one per CU (4M keys take
// 512 8192-key tiles, 22% faster per sort than 1024 4096-key tiles).
constexpr uint64_t kMinTiles = LRS_MIN_TILES;
// Rows up to this length are sorted whole inside one workgroup's LDS.
constexpr uint64_t kResidentMax = 8192;

// The largest tile shape with at least kMinTiles tiles and at most 1/32 of
// its elements past row ends (rows of 65536 take eight 8192-key tiles, not
// five 15360-key tiles with 15% padding).
int choose_tile_cfg(uint64_t rows, uint64_t row_len, bool key64) {
    for (int c = 2; c >= 1; --c) {
        const uint64_t tile = tile_cfg_of(key64, c).tile;
        const uint64_t tiles = rows * ((row_len + tile - 1) / tile);
        const uint64_t padded = tiles * tile;
        if (tiles >= kMinTiles && (padded - rows * row_len) * 32 <= padded) return c;
    }
    return 0;
}
constexpr uint64_t kAlign = 256;
#ifndef LRS_HIST_BLOCKS
#define LRS_HIST_BLOCKS 512
#endif
// Histogram workgroups per launch: 1024 threads and 128 KB of LDS counters
// each, so one per CU at a time (measured on 2^28 keys against 256 and, with
// smaller workgroups and fewer copies, 640 to 5120).
constexpr uint32_t kHistTargetBlocks = LRS_HIST_BLOCKS;
#ifndef LRS_HIST_MIN_CHUNK
#define LRS_HIST_MIN_CHUNK 16384
#endif
// Fewest keys per histogram workgroup: each workgroup adds its counters to the
// row's histogram with global atomics, and on 4M keys 1024 workgroups spent
// more time on those than on reading (26 us against 16 us with 256).
constexpr uint32_t kHistMinChunk = LRS_HIST_MIN_CHUNK;

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
inline uint64_t cdiv(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

bool digit_bits_ok(int b) { return b == 1 || b == 2 || b == 4 || b == 8; }

// ---------------------------------------------------------------- timing

struct Timing {
    bool on = false;
    std::vector<hipEvent_t> pool;  // pairs: start, stop
    std::vector<int> kind;
    size_t used = 0;
};
Timing g_timing;
constexpr size_t kMaxTimed = 65536;

// Brackets one launch with events when timing is on.  Returns the pair index or -1.
struct TimedLaunch {
    int idx = -1;
    hipStream_t s;
    TimedLaunch(int kind, hipStream_t stream) : s(stream) {
        if (!g_timing.on || g_timing.used >= kMaxTimed) return;
        const size_t i = g_timing.used;
        if (g_timing.pool.size() < 2 * (i + 1)) {
            hipEvent_t a, b;
            if (hipEventCreate(&a) != hipSuccess) return;
            if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
            g_timing.pool.push_back(a);
            g_timing.pool.push_back(b);
        }
        if (hipEventRecord(g_timing.pool[2 * i], s) != hipSuccess) return;
        g_timing.kind.resize(i + 1);
        g_timing.kind[i] = kind;
        g_timing.used = i + 1;
        idx = static_cast<int>(i);
    }
    void done() {
        if (idx >= 0) (void)hipEventRecord(g_timing.pool[2 * idx + 1], s);
    }
};

// Polls of an unpublished look-back word before a tile counts its prefix from
// the keys (about 1 us each, so the default is tens of milliseconds: far beyond
// any wait of a running sort, and only a guarantee against waiting forever).
constexpr uint32_t kDefaultSpinLimit = 1u << 16;
uint32_t g_spin_limit = kDefaultSpinLimit;

// Scan strategy of single-row sorts (LRS_SCAN_*); segmented rows always use the look-back.
int g_scan_strategy = LRS_SCAN_LOOKBACK;
// Partitions of the reduce-then-scan path: two workgroups per CU.
constexpr uint64_t kPartitions = 512;

// ------------------------------------------------------------ planning

struct Plan {
    uint64_t rows = 1;
    uint64_t row_len = 0;
    int passes = 0;
    int b = 8;
    int begin_bit = 0;
    int end_bit = 32;
    bool resident = false;          // whole row sorted in one workgroup, no workspace
    int tile_cfg = 0;
    uint32_t tiles_per_row = 0;
    uint64_t num_tiles = 0;
    bool wide_status = false;       // 64-bit look-back words and store addresses (see make_plan)
    uint32_t hist_chunks_per_row = 0;
    // workspace layout (byte offsets)
    uint64_t off_hist = 0, hist_words = 0;
    uint64_t off_counters = 0, counter_words = 0;
    uint64_t off_status[2] = {0, 0}, status_bytes = 0;
    uint64_t off_alt_keys = 0, off_alt_vals = 0, off_idx[2] = {0, 0};
    uint64_t total = 0;
};

// kind: 0 keys, 1 pairs, 2 segmented
// kind: 0 keys, 1 pairs, 2 segmented; key_bytes: 4 or 8 (segmented keys are 2 bytes)
Plan make_plan(uint64_t rows, uint64_t row_len, int begin_bit, int end_bit, int b, int kind, int key_bytes = 4) {
    Plan p;
    const bool key64 = key_bytes == 8;
    p.rows = rows;
    p.row_len = row_len;
    p.b = b;
    p.begin_bit = begin_bit;
    p.end_bit = end_bit;
    p.passes = static_cast<int>(cdiv(static_cast<uint64_t>(end_bit - begin_bit), b));
    const uint64_t R = 1ull << b;
    p.tile_cfg = choose_tile_cfg(rows, row_len, key64);
    p.tiles_per_row = static_cast<uint32_t>(cdiv(row_len, tile_cfg_of(key64, p.tile_cfg).tile));
    p.num_tiles = rows * p.tiles_per_row;
    // A row needs the wide sweep (64-bit look-back words, 64-bit store
    // addresses) once its byte offsets pass what a 32-bit buffer offset
    // reaches (2^32 bytes) or its counts pass the 30-bit count of a 32-bit
    // look-back word: from 2^30 elements of 4 bytes, and from 2^29 for 8-byte
    // keys and for row sorts (int64 index out).
    const uint64_t widest = (kind == 2) ? 8 : static_cast<uint64_t>(key_bytes);
    p.wide_status = row_len * widest >= (1ull << 32) || row_len >= (1ull << 30);

    // histogram: about kHistTargetBlocks workgroups in all, at least
    // kHistMinChunk keys each
    p.hist_chunks_per_row = static_cast<uint32_t>(std::max<uint64_t>(
        1, std::min<uint64_t>(cdiv(row_len, kHistMinChunk), cdiv(kHistTargetBlocks, rows))));

    const uint64_t keysz = (kind == 2) ? 2 : static_cast<uint64_t>(key_bytes);
    const uint64_t n = rows * row_len;
    uint64_t off = 0;
    p.off_hist = off;
    p.hist_words = rows * p.passes * R;
    off = align_up(off + 4 * p.hist_words, kAlign);
    p.off_counters = off;
    p.counter_words = static_cast<uint64_t>(p.passes) * kXcds;
    off = align_up(off + 4 * p.counter_words, kAlign);
    p.status_bytes = p.num_tiles * R * (p.wide_status ? 8 : 4);
    const int status_bufs = p.passes > 1 ? 2 : 1;
    for (int i = 0; i < status_bufs; ++i) {
        p.off_status[i] = off;
        off = align_up(off + p.status_bytes, kAlign);
    }
    if (p.passes > 1) {
        p.off_alt_keys = off;
        off = align_up(off + n * keysz, kAlign);
        if (kind == 1) {
            p.off_alt_vals = off;
            off = align_up(off + n * 4, kAlign);
        }
        if (kind == 2) {
            p.off_idx[0] = off;
            off = align_up(off + n * 4, kAlign);
            if (p.passes > 2) {
                p.off_idx[1] = off;
                off = align_up(off + n * 4, kAlign);
            }
        }
    }
    p.total = off;
    if (row_len <= kResidentMax && !key64) {
        p.resident = true;
        p.total = 0;
    }
    return p;
}

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// ------------------------------------------------------------ launches

// Whole-row resident sort, timed as kind 4.
template <int KK, int PK>
hipError_t resident(int b, const ResidentArgs &a, uint64_t rows, uint64_t row_len, hipStream_t s) {
    TimedLaunch t(4, s);
    const hipError_t e = launch_resident<KK, PK>(b, a, rows, row_len, s);
    t.done();
    return e;
}

hipError_t launch_clear(const Plan &p, uint8_t *ws, bool need_hist, hipStream_t s) {
    ClearArgs c{};
    c.p[0] = need_hist ? reinterpret_cast<uint32_t *>(ws + p.off_hist) : nullptr;
    c.words[0] = p.hist_words;
    c.p[1] = reinterpret_cast<uint32_t *>(ws + p.off_counters);
    c.words[1] = p.counter_words;
    c.p[2] = reinterpret_cast<uint32_t *>(ws + p.off_status[0]);
    c.words[2] = p.status_bytes / 4;
    const uint64_t words = std::max<uint64_t>(c.words[0] * need_hist, c.words[2]);
    const uint32_t blocks = static_cast<uint32_t>(std::min<uint64_t>(2048, std::max<uint64_t>(1, cdiv(words / 4, kBlock))));
    TimedLaunch t(0, s);
    clear_kernel<<<blocks, kBlock, 0, s>>>(c);
    hipError_t e = hipGetLastError();
    t.done();
    return e;
}

hipError_t launch_histogram(const Plan &p, const void *keys, uint32_t *hist, int kk, uint64_t flip, uint64_t flip_neg,
                            bool accumulate, hipStream_t s) {
    HistArgs h{};
    h.keys = keys;
    h.hist = hist;
    h.row_len = static_cast<uint32_t>(p.row_len);
    h.chunks_per_row = p.hist_chunks_per_row;
    h.passes = static_cast<uint32_t>(p.passes);
    h.begin_bit = static_cast<uint32_t>(p.begin_bit);
    h.end_bit = static_cast<uint32_t>(p.end_bit);
    h.flip = flip;
    h.flip_neg = flip_neg;
    h.atomic = accumulate ? 1u : 0u;
    const uint64_t blocks = p.rows * p.hist_chunks_per_row;
    TimedLaunch t(1, s);
    hipError_t e = (kk == kKeyU32)   ? launch_hist<kKeyU32>(p.b, h, static_cast<uint32_t>(blocks), s)
                   : (kk == kKeyX32) ? launch_hist<kKeyX32>(p.b, h, static_cast<uint32_t>(blocks), s)
                   : (kk == kKeyU64) ? launch_hist<kKeyU64>(p.b, h, static_cast<uint32_t>(blocks), s)
                   : (kk == kKeyX64) ? launch_hist<kKeyX64>(p.b, h, static_cast<uint32_t>(blocks), s)
                                     : launch_hist<kKeyF16>(p.b, h, static_cast<uint32_t>(blocks), s);
    t.done();
    return e;
}

SweepArgs pass_args(const Plan &p, uint8_t *ws, int pass) {
    SweepArgs a{};
    const uint64_t R = 1ull << p.b;
    a.hist = reinterpret_cast<const uint32_t *>(ws + p.off_hist) + static_cast<uint64_t>(pass) * R;
    a.hist_row_stride = static_cast<uint32_t>(p.passes * R);
    a.status = ws + p.off_status[pass & 1];
    a.status_next = (pass + 1 < p.passes) ? ws + p.off_status[(pass + 1) & 1] : nullptr;
    a.tile_counter = reinterpret_cast<uint32_t *>(ws + p.off_counters) + static_cast<uint64_t>(pass) * kXcds;
    a.row_len = static_cast<uint32_t>(p.row_len);
    a.tiles_per_row = p.tiles_per_row;
    a.num_tiles = static_cast<uint32_t>(p.num_tiles);
    const int shift = p.begin_bit + pass * p.b;
    const int width = std::min(p.b, p.end_bit - shift);
    a.shift = static_cast<uint32_t>(shift);
    a.digit_mask = (1u << width) - 1u;
    a.flip = 0;
    a.flip_neg = 0;
    a.spin_limit = g_spin_limit;
    return a;
}

// Buffer that pass `pass` writes: the last pass writes the caller's output,
// earlier passes alternate backwards between the spare buffer and the output.
template <typename T>
T *pass_dst(int pass, int passes, T *out, T *alt) {
    return ((passes - 1 - pass) % 2 == 0) ? out : alt;
}

// Kernel key kind and transform masks of a (key type, direction); false for an
// unknown key type.  The masks give each type's order-preserving u32 image and
// complement it for descending order (see KeyTraits<kKeyX32>).
bool key_transform(int key_type, int descending, int &kk, uint64_t &flip, uint64_t &flip_neg) {
    const uint64_t c = descending ? ~0ull : 0ull;
    const uint64_t c32 = c & 0xFFFFFFFFull;
    const uint64_t top64 = 1ull << 63;
    switch (key_type) {
        case LRS_KEY_U32: kk = descending ? kKeyX32 : kKeyU32; flip = c32; flip_neg = c32; return true;
        case LRS_KEY_I32: kk = kKeyX32; flip = 0x80000000ull ^ c32; flip_neg = 0x80000000ull ^ c32; return true;
        case LRS_KEY_F32: kk = kKeyX32; flip = 0x80000000ull ^ c32; flip_neg = 0xFFFFFFFFull ^ c32; return true;
        case LRS_KEY_U64: kk = descending ? kKeyX64 : kKeyU64; flip = c; flip_neg = c; return true;
        case LRS_KEY_I64: kk = kKeyX64; flip = top64 ^ c; flip_neg = top64 ^ c; return true;
        case LRS_KEY_F64: kk = kKeyX64; flip = top64 ^ c; flip_neg = ~0ull ^ c; return true;
        default: return false;
    }
}

bool key_type_is_64(int key_type) {
    return key_type == LRS_KEY_U64 || key_type == LRS_KEY_I64 || key_type == LRS_KEY_F64;
}

// Reduce-then-scan passes (CUDA Handbook ch.16: count, scan the counts, scatter;
// 100 Days of GPU, Day 35: persistent blocks walking their tiles in order): per
// pass, an upsweep counts the digit over each of up to 512 partitions of whole
// tiles, one workgroup scans those counts into start offsets, and the sweep
// sorts each partition's tiles in order from them.  No histogram kernel, no
// look-back; the upsweep reads the keys once more per pass.
int sort_32_reduce_then_scan(const Plan &p, int kk, uint64_t flip, uint64_t flip_neg, bool pairs,
                             const uint32_t *keys_in, const uint32_t *vals_in, uint32_t *keys_out,
                             uint32_t *vals_out, uint8_t *ws, hipStream_t s) {
    const uint64_t part_tiles = cdiv(p.num_tiles, std::min<uint64_t>(p.num_tiles, kPartitions));
    const uint64_t partitions = cdiv(p.num_tiles, part_tiles);
    uint32_t *counts = reinterpret_cast<uint32_t *>(ws + p.off_status[0]);  // partitions x R <= tiles x R
    uint32_t *alt_k = reinterpret_cast<uint32_t *>(ws + p.off_alt_keys);
    uint32_t *alt_v = reinterpret_cast<uint32_t *>(ws + p.off_alt_vals);
    const uint32_t *src_k = keys_in;
    const uint32_t *src_v = vals_in;
    for (int pass = 0; pass < p.passes; ++pass) {
        SweepArgs a = pass_args(p, ws, pass);
        PartArgs pa{};
        pa.keys = src_k;
        pa.counts = counts;
        pa.n = static_cast<uint32_t>(p.row_len);
        pa.part_len = static_cast<uint32_t>(part_tiles * tile_cfg_of(false, p.tile_cfg).tile);
        pa.partitions = static_cast<uint32_t>(partitions);
        pa.shift = a.shift;
        pa.digit_mask = a.digit_mask;
        pa.flip = flip;
        pa.flip_neg = flip_neg;
        {
            TimedLaunch t(1, s);
            const hipError_t e = (kk == kKeyU32) ? launch_partition_counts<kKeyU32>(p.b, pa, s)
                                                 : launch_partition_counts<kKeyX32>(p.b, pa, s);
            t.done();
            if (e != hipSuccess) return LRS_ERR_HIP;
        }
        uint32_t *dk = pass_dst(pass, p.passes, keys_out, alt_k);
        a.keys_in = src_k;
        a.keys_out = dk;
        a.flip = flip;
        a.flip_neg = flip_neg;
        a.part_offsets = counts;
        a.part_tiles = static_cast<uint32_t>(part_tiles);
        hipError_t e;
        TimedLaunch t(2, s);
        if (pairs) {
            uint32_t *dv = pass_dst(pass, p.passes, vals_out, alt_v);
            a.vals_in = src_v;
            a.vals_out = dv;
            e = (kk == kKeyU32) ? launch_sweep<kKeyU32, kPayU32, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, s)
                                : launch_sweep<kKeyX32, kPayU32, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, s);
            src_v = dv;
        } else {
            e = (kk == kKeyU32) ? launch_sweep<kKeyU32, kPayNone, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, s)
                                : launch_sweep<kKeyX32, kPayNone, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, s);
        }
        t.done();
        if (e != hipSuccess) return LRS_ERR_HIP;
        src_k = dk;
    }
    return LRS_OK;
}

// Keys of 32 bits: u32 as they are (KK = kKeyU32), anything else through the
// two-mask transform (KK = kKeyX32).
int sort_32(int kk, uint64_t flip, uint64_t flip_neg, bool pairs, const uint32_t *keys_in,
            const uint32_t *vals_in, uint32_t *keys_out, uint32_t *vals_out, uint64_t n, int begin_bit,
            int end_bit, int b, void *workspace, size_t ws_bytes, void *stream) {
    if (!digit_bits_ok(b)) return LRS_ERR_DIGIT_BITS;
    if (begin_bit < 0 || end_bit > 32 || begin_bit >= end_bit) return LRS_ERR_BIT_RANGE;
    if (n > LRS_MAX_KEYS) return LRS_ERR_SIZE;
    if (n == 0) return LRS_OK;
    const Plan p = make_plan(1, n, begin_bit, end_bit, b, pairs ? 1 : 0);
    if (!keys_in || !keys_out || (pairs && (!vals_in || !vals_out)) || (p.total && !workspace))
        return LRS_ERR_NULL_POINTER;
    if (misaligned(keys_in, 4) || misaligned(keys_out, 4) || misaligned(workspace, 256) ||
        (pairs && (misaligned(vals_in, 4) || misaligned(vals_out, 4))))
        return LRS_ERR_ALIGNMENT;
    if (ws_bytes < p.total) return LRS_ERR_WORKSPACE_TOO_SMALL;
    const uint64_t kb = 4 * n;
    if (overlaps(keys_out, kb, keys_in, kb) || overlaps(keys_out, kb, workspace, p.total) ||
        (pairs && (overlaps(vals_out, kb, vals_in, kb) || overlaps(vals_out, kb, keys_in, kb) ||
                   overlaps(keys_out, kb, vals_in, kb) || overlaps(vals_out, kb, keys_out, kb) ||
                   overlaps(vals_out, kb, workspace, p.total))))
        return LRS_ERR_ALIASING;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.resident) {
        ResidentArgs r{};
        r.keys_in = keys_in;
        r.keys_out = keys_out;
        r.vals_in = vals_in;
        r.vals_out = vals_out;
        r.row_len = static_cast<uint32_t>(n);
        r.begin_bit = static_cast<uint32_t>(begin_bit);
        r.end_bit = static_cast<uint32_t>(end_bit);
        r.flip = flip;
        r.flip_neg = flip_neg;
        hipError_t e;
        if (kk == kKeyU32)
            e = pairs ? resident<kKeyU32, kResU32>(b, r, 1, n, s) : resident<kKeyU32, kResNone>(b, r, 1, n, s);
        else
            e = pairs ? resident<kKeyX32, kResU32>(b, r, 1, n, s) : resident<kKeyX32, kResNone>(b, r, 1, n, s);
        return e == hipSuccess ? LRS_OK : LRS_ERR_HIP;
    }
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    if (g_scan_strategy == LRS_SCAN_REDUCE_THEN_SCAN)
        return sort_32_reduce_then_scan(p, kk, flip, flip_neg, pairs, keys_in, vals_in, keys_out, vals_out, ws, s);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + p.off_hist);
    if (launch_clear(p, ws, p.hist_chunks_per_row > 1, s) != hipSuccess) return LRS_ERR_HIP;
    if (launch_histogram(p, keys_in, hist, kk, flip, flip_neg, p.hist_chunks_per_row > 1, s) != hipSuccess)
        return LRS_ERR_HIP;

    uint32_t *alt_k = reinterpret_cast<uint32_t *>(ws + p.off_alt_keys);
    uint32_t *alt_v = reinterpret_cast<uint32_t *>(ws + p.off_alt_vals);
    const uint32_t *src_k = keys_in;
    const uint32_t *src_v = vals_in;
    for (int pass = 0; pass < p.passes; ++pass) {
        SweepArgs a = pass_args(p, ws, pass);
        uint32_t *dk = pass_dst(pass, p.passes, keys_out, alt_k);
        a.keys_in = src_k;
        a.keys_out = dk;
        a.flip = flip;
        a.flip_neg = flip_neg;
        hipError_t e;
        TimedLaunch t(2, s);
        if (pairs) {
            uint32_t *dv = pass_dst(pass, p.passes, vals_out, alt_v);
            a.vals_in = src_v;
            a.vals_out = dv;
            e = (kk == kKeyU32) ? launch_sweep<kKeyU32, kPayU32, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, s)
                                : launch_sweep<kKeyX32, kPayU32, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, s);
            src_v = dv;
        } else {
            e = (kk == kKeyU32) ? launch_sweep<kKeyU32, kPayNone, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, s)
                                : launch_sweep<kKeyX32, kPayNone, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, s);
        }
        t.done();
        if (e != hipSuccess) return LRS_ERR_HIP;
        src_k = dk;
    }
    return LRS_OK;
}

// Keys of 64 bits (u64 as they are, anything else through the two-mask
// transform): the look-back path with 64-bit tile shapes; no whole-row
// resident sort and no reduce-then-scan.
int sort_64(int kk, uint64_t flip, uint64_t flip_neg, bool pairs, const uint64_t *keys_in,
            const uint32_t *vals_in, uint64_t *keys_out, uint32_t *vals_out, uint64_t n, int begin_bit,
            int end_bit, int b, void *workspace, size_t ws_bytes, void *stream) {
    if (!digit_bits_ok(b)) return LRS_ERR_DIGIT_BITS;
    if (begin_bit < 0 || end_bit > 64 || begin_bit >= end_bit) return LRS_ERR_BIT_RANGE;
    if (n > LRS_MAX_KEYS) return LRS_ERR_SIZE;
    if (n == 0) return LRS_OK;
    const Plan p = make_plan(1, n, begin_bit, end_bit, b, pairs ? 1 : 0, 8);
    if (!keys_in || !keys_out || (pairs && (!vals_in || !vals_out)) || !workspace) return LRS_ERR_NULL_POINTER;
    if (misaligned(keys_in, 8) || misaligned(keys_out, 8) || misaligned(workspace, 256) ||
        (pairs && (misaligned(vals_in, 4) || misaligned(vals_out, 4))))
        return LRS_ERR_ALIGNMENT;
    if (ws_bytes < p.total) return LRS_ERR_WORKSPACE_TOO_SMALL;
    const uint64_t kb = 8 * n, vb = 4 * n;
    if (overlaps(keys_out, kb, keys_in, kb) || overlaps(keys_out, kb, workspace, p.total) ||
        (pairs && (overlaps(vals_out, vb, vals_in, vb) || overlaps(vals_out, vb, keys_in, kb) ||
                   overlaps(keys_out, kb, vals_in, vb) || overlaps(vals_out, vb, keys_out, kb) ||
                   overlaps(vals_out, vb, workspace, p.total))))
        return LRS_ERR_ALIASING;

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + p.off_hist);
    if (launch_clear(p, ws, p.hist_chunks_per_row > 1, s) != hipSuccess) return LRS_ERR_HIP;
    if (launch_histogram(p, keys_in, hist, kk, flip, flip_neg, p.hist_chunks_per_row > 1, s) != hipSuccess)
        return LRS_ERR_HIP;
    uint64_t *alt_k = reinterpret_cast<uint64_t *>(ws + p.off_alt_keys);
    uint32_t *alt_v = reinterpret_cast<uint32_t *>(ws + p.off_alt_vals);
    const uint64_t *src_k = keys_in;
    const uint32_t *src_v = vals_in;
    for (int pass = 0; pass < p.passes; ++pass) {
        SweepArgs a = pass_args(p, ws, pass);
        uint64_t *dk = pass_dst(pass, p.passes, keys_out, alt_k);
        a.keys_in = src_k;
        a.keys_out = dk;
        a.flip = flip;
        a.flip_neg = flip_neg;
        hipError_t e;
        TimedLaunch t(2, s);
        if (pairs) {
            uint32_t *dv = pass_dst(pass, p.passes, vals_out, alt_v);
            a.vals_in = src_v;
            a.vals_out = dv;
            e = (kk == kKeyU64) ? launch_sweep<kKeyU64, kPayU32, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, s)
                                : launch_sweep<kKeyX64, kPayU32, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, s);
            src_v = dv;
        } else {
            e = (kk == kKeyU64) ? launch_sweep<kKeyU64, kPayNone, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, s)
                                : launch_sweep<kKeyX64, kPayNone, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, s);
        }
        t.done();
        if (e != hipSuccess) return LRS_ERR_HIP;
        src_k = dk;
    }
    return LRS_OK;
}

}  // namespace
}  // namespace lrs

using namespace lrs;

extern "C" {

size_t radix_sort_workspace_size(uint64_t n, int begin_bit, int end_bit, int digit_bits,
                                 int with_values) {
    if (!digit_bits_ok(digit_bits) || begin_bit < 0 || end_bit > 32 || begin_bit >= end_bit ||
        n == 0 || n > LRS_MAX_KEYS)
        return 0;
    return static_cast<size_t>(make_plan(1, n, begin_bit, end_bit, digit_bits, with_values ? 1 : 0).total);
}

int radix_sort_keys(const uint32_t *keys_in, uint32_t *keys_out, uint64_t n, int begin_bit,
                    int end_bit, int digit_bits, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return sort_32(kKeyU32, 0, 0, false, keys_in, nullptr, keys_out, nullptr, n, begin_bit, end_bit,
                   digit_bits, workspace, workspace_bytes, stream);
}

int radix_sort_pairs(const uint32_t *keys_in, const uint32_t *vals_in, uint32_t *keys_out,
                     uint32_t *vals_out, uint64_t n, int begin_bit, int end_bit, int digit_bits,
                     void *workspace, size_t workspace_bytes, void *stream) {
    return sort_32(kKeyU32, 0, 0, true, keys_in, vals_in, keys_out, vals_out, n, begin_bit, end_bit,
                   digit_bits, workspace, workspace_bytes, stream);
}

size_t radix_sort_typed_workspace_size(uint64_t n, int key_type, int begin_bit, int end_bit, int digit_bits,
                                       int with_values) {
    int kk;
    uint64_t flip, flip_neg;
    if (!key_transform(key_type, 0, kk, flip, flip_neg)) return 0;
    const int key_bits = key_type_is_64(key_type) ? 64 : 32;
    if (!digit_bits_ok(digit_bits) || begin_bit < 0 || end_bit > key_bits || begin_bit >= end_bit || n == 0 ||
        n > LRS_MAX_KEYS)
        return 0;
    return static_cast<size_t>(
        make_plan(1, n, begin_bit, end_bit, digit_bits, with_values ? 1 : 0, key_bits / 8).total);
}

int radix_sort_keys_typed(const void *keys_in, void *keys_out, uint64_t n, int key_type, int descending,
                          int begin_bit, int end_bit, int digit_bits, void *workspace,
                          size_t workspace_bytes, void *stream) {
    int kk;
    uint64_t flip, flip_neg;
    if (!key_transform(key_type, descending, kk, flip, flip_neg)) return LRS_ERR_DTYPE;
    if (key_type_is_64(key_type))
        return sort_64(kk, flip, flip_neg, false, static_cast<const uint64_t *>(keys_in), nullptr,
                       static_cast<uint64_t *>(keys_out), nullptr, n, begin_bit, end_bit, digit_bits, workspace,
                       workspace_bytes, stream);
    return sort_32(kk, flip, flip_neg, false, static_cast<const uint32_t *>(keys_in), nullptr,
                   static_cast<uint32_t *>(keys_out), nullptr, n, begin_bit, end_bit, digit_bits, workspace,
                   workspace_bytes, stream);
}

int radix_sort_pairs_typed(const void *keys_in, const uint32_t *vals_in, void *keys_out, uint32_t *vals_out,
                           uint64_t n, int key_type, int descending, int begin_bit, int end_bit,
                           int digit_bits, void *workspace, size_t workspace_bytes, void *stream) {
    int kk;
    uint64_t flip, flip_neg;
    if (!key_transform(key_type, descending, kk, flip, flip_neg)) return LRS_ERR_DTYPE;
    if (key_type_is_64(key_type))
        return sort_64(kk, flip, flip_neg, true, static_cast<const uint64_t *>(keys_in), vals_in,
                       static_cast<uint64_t *>(keys_out), vals_out, n, begin_bit, end_bit, digit_bits, workspace,
                       workspace_bytes, stream);
    return sort_32(kk, flip, flip_neg, true, static_cast<const uint32_t *>(keys_in), vals_in,
                   static_cast<uint32_t *>(keys_out), vals_out, n, begin_bit, end_bit, digit_bits, workspace,
                   workspace_bytes, stream);
}

size_t segmented_row_sort_workspace_size(int64_t rows, int64_t n, int digit_bits) {
    if (!digit_bits_ok(digit_bits) || rows <= 0 || n <= 0 ||
        static_cast<uint64_t>(n) > LRS_MAX_ROW_LEN ||
        static_cast<uint64_t>(rows) * static_cast<uint64_t>(n) >= (1ull << 40))
        return 0;
    return static_cast<size_t>(make_plan(rows, n, 0, 16, digit_bits, 2).total);
}

int segmented_row_sort(const uint16_t *vals_in, uint16_t *vals_out, int64_t *idx_out,
                       int64_t rows, int64_t n, int dtype, int descending, int digit_bits,
                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!digit_bits_ok(digit_bits)) return LRS_ERR_DIGIT_BITS;
    if (dtype != LRS_DTYPE_FP16 && dtype != LRS_DTYPE_BF16) return LRS_ERR_DTYPE;
    if (rows < 0 || n < 0 || static_cast<uint64_t>(n) > LRS_MAX_ROW_LEN ||
        (rows > 0 && static_cast<uint64_t>(rows) * static_cast<uint64_t>(n) >= (1ull << 40)))
        return LRS_ERR_SIZE;
    if (rows == 0 || n == 0) return LRS_OK;
    const Plan p = make_plan(rows, n, 0, 16, digit_bits, 2);
    if (!vals_in || !vals_out || !idx_out || (p.total && !workspace)) return LRS_ERR_NULL_POINTER;
    if (misaligned(vals_in, 2) || misaligned(vals_out, 2) || misaligned(idx_out, 8) ||
        misaligned(workspace, 256))
        return LRS_ERR_ALIGNMENT;
    if (p.num_tiles > 0x7FFFFFFFull || p.rows * p.hist_chunks_per_row > 0x7FFFFFFFull) return LRS_ERR_SIZE;
    if (workspace_bytes < p.total) return LRS_ERR_WORKSPACE_TOO_SMALL;
    const uint64_t cnt = static_cast<uint64_t>(rows) * n;
    if (overlaps(vals_out, 2 * cnt, vals_in, 2 * cnt) || overlaps(idx_out, 8 * cnt, vals_in, 2 * cnt) ||
        overlaps(idx_out, 8 * cnt, vals_out, 2 * cnt) || overlaps(vals_out, 2 * cnt, workspace, p.total) ||
        overlaps(idx_out, 8 * cnt, workspace, p.total))
        return LRS_ERR_ALIASING;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t flip = descending ? 0xFFFFu : 0u;
    if (p.resident) {
        if (rows > 0x7FFFFFFF) return LRS_ERR_SIZE;
        ResidentArgs r{};
        r.keys_in = vals_in;
        r.keys_out = vals_out;
        r.vals_out = idx_out;
        r.row_len = static_cast<uint32_t>(n);
        r.begin_bit = 0;
        r.end_bit = 16;
        r.flip = flip;
        const hipError_t e = resident<kKeyF16, kResIndex>(digit_bits, r, rows, n, s);
        return e == hipSuccess ? LRS_OK : LRS_ERR_HIP;
    }
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + p.off_hist);
    if (launch_clear(p, ws, p.hist_chunks_per_row > 1, s) != hipSuccess) return LRS_ERR_HIP;
    if (launch_histogram(p, vals_in, hist, kKeyF16, flip, 0, p.hist_chunks_per_row > 1, s) != hipSuccess) return LRS_ERR_HIP;

    uint16_t *alt_k = reinterpret_cast<uint16_t *>(ws + p.off_alt_keys);
    uint32_t *idx[2] = {reinterpret_cast<uint32_t *>(ws + p.off_idx[0]),
                        reinterpret_cast<uint32_t *>(ws + p.off_idx[1])};
    const uint16_t *src_k = vals_in;
    for (int pass = 0; pass < p.passes; ++pass) {
        SweepArgs a = pass_args(p, ws, pass);
        a.flip = flip;
        uint16_t *dk = pass_dst(pass, p.passes, vals_out, alt_k);
        a.keys_in = src_k;
        a.keys_out = dk;
        hipError_t e;
        TimedLaunch t(2, s);
        if (pass == 0) {
            a.vals_in = nullptr;
            a.vals_out = idx[0];
            e = launch_sweep<kKeyF16, kPayIdxFirst, false>(digit_bits, a, p.tile_cfg, p.wide_status, p.num_tiles, s);
        } else if (pass + 1 < p.passes) {
            a.vals_in = idx[(pass - 1) & 1];
            a.vals_out = idx[pass & 1];
            e = launch_sweep<kKeyF16, kPayU32, false>(digit_bits, a, p.tile_cfg, p.wide_status, p.num_tiles, s);
        } else {
            a.vals_in = idx[(pass - 1) & 1];
            a.vals_out = idx_out;
            e = launch_sweep<kKeyF16, kPayIdxLast, false>(digit_bits, a, p.tile_cfg, p.wide_status, p.num_tiles, s);
        }
        t.done();
        if (e != hipSuccess) return LRS_ERR_HIP;
        src_k = dk;
    }
    return LRS_OK;
}

int segmented_row_sort_pairs(const uint16_t *vals_in, const uint32_t *pay_in, uint16_t *vals_out,
                             uint32_t *pay_out, int64_t rows, int64_t n, int dtype, int descending,
                             int digit_bits, void *workspace, size_t workspace_bytes, void *stream) {
    if (!digit_bits_ok(digit_bits)) return LRS_ERR_DIGIT_BITS;
    if (dtype != LRS_DTYPE_FP16 && dtype != LRS_DTYPE_BF16) return LRS_ERR_DTYPE;
    if (rows < 0 || n < 0 || static_cast<uint64_t>(n) > LRS_MAX_ROW_LEN ||
        (rows > 0 && static_cast<uint64_t>(rows) * static_cast<uint64_t>(n) >= (1ull << 40)))
        return LRS_ERR_SIZE;
    if (rows == 0 || n == 0) return LRS_OK;
    const Plan p = make_plan(rows, n, 0, 16, digit_bits, 2);
    if (!vals_in || !vals_out || !pay_in || !pay_out || (p.total && !workspace)) return LRS_ERR_NULL_POINTER;
    if (misaligned(vals_in, 2) || misaligned(vals_out, 2) || misaligned(pay_in, 4) || misaligned(pay_out, 4) ||
        misaligned(workspace, 256))
        return LRS_ERR_ALIGNMENT;
    if (p.num_tiles > 0x7FFFFFFFull || p.rows * p.hist_chunks_per_row > 0x7FFFFFFFull) return LRS_ERR_SIZE;
    if (workspace_bytes < p.total) return LRS_ERR_WORKSPACE_TOO_SMALL;
    const uint64_t cnt = static_cast<uint64_t>(rows) * n;
    if (overlaps(vals_out, 2 * cnt, vals_in, 2 * cnt) || overlaps(vals_out, 2 * cnt, pay_in, 4 * cnt) ||
        overlaps(pay_out, 4 * cnt, vals_in, 2 * cnt) || overlaps(pay_out, 4 * cnt, pay_in, 4 * cnt) ||
        overlaps(pay_out, 4 * cnt, vals_out, 2 * cnt) || overlaps(vals_out, 2 * cnt, workspace, p.total) ||
        overlaps(pay_out, 4 * cnt, workspace, p.total))
        return LRS_ERR_ALIASING;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t flip = descending ? 0xFFFFu : 0u;
    if (p.resident) {
        if (rows > 0x7FFFFFFF) return LRS_ERR_SIZE;
        ResidentArgs r{};
        r.keys_in = vals_in;
        r.keys_out = vals_out;
        r.vals_in = pay_in;
        r.vals_out = pay_out;
        r.row_len = static_cast<uint32_t>(n);
        r.begin_bit = 0;
        r.end_bit = 16;
        r.flip = flip;
        const hipError_t e = resident<kKeyF16, kResU32>(digit_bits, r, rows, n, s);
        return e == hipSuccess ? LRS_OK : LRS_ERR_HIP;
    }
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + p.off_hist);
    if (launch_clear(p, ws, p.hist_chunks_per_row > 1, s) != hipSuccess) return LRS_ERR_HIP;
    if (launch_histogram(p, vals_in, hist, kKeyF16, flip, 0, p.hist_chunks_per_row > 1, s) != hipSuccess) return LRS_ERR_HIP;
    uint16_t *alt_k = reinterpret_cast<uint16_t *>(ws + p.off_alt_keys);
    uint32_t *alt_p = reinterpret_cast<uint32_t *>(ws + p.off_idx[0]);
    const uint16_t *src_k = vals_in;
    const uint32_t *src_p = pay_in;
    for (int pass = 0; pass < p.passes; ++pass) {
        SweepArgs a = pass_args(p, ws, pass);
        a.flip = flip;
        uint16_t *dk = pass_dst(pass, p.passes, vals_out, alt_k);
        uint32_t *dp = pass_dst(pass, p.passes, pay_out, alt_p);
        a.keys_in = src_k;
        a.keys_out = dk;
        a.vals_in = src_p;
        a.vals_out = dp;
        TimedLaunch t(2, s);
        const hipError_t e = launch_sweep<kKeyF16, kPayU32, false>(digit_bits, a, p.tile_cfg, p.wide_status, p.num_tiles, s);
        t.done();
        if (e != hipSuccess) return LRS_ERR_HIP;
        src_k = dk;
        src_p = dp;
    }
    return LRS_OK;
}

int radix_sort_digit_histograms(const uint32_t *keys, uint64_t n, int begin_bit, int end_bit,
                                int digit_bits, uint32_t *hist_out, void *stream) {
    if (!digit_bits_ok(digit_bits)) return LRS_ERR_DIGIT_BITS;
    if (begin_bit < 0 || end_bit > 32 || begin_bit >= end_bit) return LRS_ERR_BIT_RANGE;
    if (n > LRS_MAX_KEYS) return LRS_ERR_SIZE;
    if (!hist_out || (n && !keys)) return LRS_ERR_NULL_POINTER;
    if (misaligned(keys, 4) || misaligned(hist_out, 16)) return LRS_ERR_ALIGNMENT;
    const Plan p = make_plan(1, n ? n : 1, begin_bit, end_bit, digit_bits, 0);
    hipStream_t s = static_cast<hipStream_t>(stream);
    ClearArgs c{};
    c.p[0] = hist_out;
    c.words[0] = p.hist_words;
    {
        TimedLaunch t(0, s);
        clear_kernel<<<1, kBlock, 0, s>>>(c);
        hipError_t e = hipGetLastError();
        t.done();
        if (e != hipSuccess) return LRS_ERR_HIP;
    }
    if (n == 0) return LRS_OK;
    return launch_histogram(p, keys, hist_out, kKeyU32, 0, 0, true, s) == hipSuccess ? LRS_OK : LRS_ERR_HIP;
}

int radix_sort_copy_probe(const void *src, void *dst, size_t bytes, void *stream) {
    if (bytes == 0) return LRS_OK;
    if (!src || !dst) return LRS_ERR_NULL_POINTER;
    if (misaligned(src, 16) || misaligned(dst, 16)) return LRS_ERR_ALIGNMENT;
    if (overlaps(src, bytes, dst, bytes)) return LRS_ERR_ALIASING;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint64_t n16 = bytes / 16;
    const uint32_t tail = static_cast<uint32_t>(bytes % 16);
    const uint32_t blocks = static_cast<uint32_t>(std::min<uint64_t>(1u << 20, std::max<uint64_t>(1, cdiv(n16, kBlock))));
    TimedLaunch t(3, s);
    copy_kernel<<<blocks, kBlock, 0, s>>>(static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n16,
                                          static_cast<const uint8_t *>(src) + n16 * 16,
                                          static_cast<uint8_t *>(dst) + n16 * 16, tail);
    hipError_t e = hipGetLastError();
    t.done();
    return e == hipSuccess ? LRS_OK : LRS_ERR_HIP;
}

int radix_sort_set_scan_strategy(int strategy) {
    if (strategy != LRS_SCAN_LOOKBACK && strategy != LRS_SCAN_REDUCE_THEN_SCAN) return -1;
    const int old = g_scan_strategy;
    g_scan_strategy = strategy;
    return old;
}

uint32_t radix_sort_set_spin_limit(uint32_t polls) {
    const uint32_t old = g_spin_limit;
    g_spin_limit = polls;
    return old;
}

int radix_sort_timing_begin(void) {
    g_timing.on = true;
    g_timing.used = 0;
    g_timing.kind.clear();
    return LRS_OK;
}

int radix_sort_timing_end(double *ms_by_kind, int *launches_by_kind) {
    for (int k = 0; k < 5; ++k) {
        if (ms_by_kind) ms_by_kind[k] = 0.0;
        if (launches_by_kind) launches_by_kind[k] = 0;
    }
    g_timing.on = false;
    for (size_t i = 0; i < g_timing.used; ++i) {
        if (hipEventSynchronize(g_timing.pool[2 * i + 1]) != hipSuccess) return LRS_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_timing.pool[2 * i], g_timing.pool[2 * i + 1]) != hipSuccess)
            return LRS_ERR_HIP;
        const int k = g_timing.kind[i];
        if (ms_by_kind) ms_by_kind[k] += ms;
        if (launches_by_kind) launches_by_kind[k] += 1;
    }
    g_timing.used = 0;
    return LRS_OK;
}

const char *radix_sort_status_string(int status) {
    switch (status) {
        case LRS_OK: return "ok";
        case LRS_ERR_NULL_POINTER: return "a required pointer is NULL";
        case LRS_ERR_BIT_RANGE: return "bit window must satisfy 0 <= begin_bit < end_bit <= key width";
        case LRS_ERR_DIGIT_BITS: return "digit_bits must be 1, 2, 4 or 8";
        case LRS_ERR_SIZE: return "element count or shape beyond the supported limit";
        case LRS_ERR_ALIASING: return "an output overlaps an input, another output or the workspace";
        case LRS_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the *_workspace_size() figure";
        case LRS_ERR_DTYPE: return "dtype must be LRS_DTYPE_FP16 or LRS_DTYPE_BF16";
        case LRS_ERR_HIP: return "the HIP runtime rejected a launch";
        case LRS_ERR_ALIGNMENT: return "a pointer is not aligned as required";
        default: return "unknown status";
    }
}

}  // extern "C"
