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
#include <mutex>
#include <vector>

#include "../../include/lsd_radix_sort.h"
#include "lrs_launch.h"

// A caller's kernel timer: start/stop event pairs and the kind of each launch.
struct lrs_timer {
    std::vector<hipEvent_t> pool;  // pairs: start, stop
    std::vector<int> kind;
    size_t used = 0;
    // tile phase records (builds with LRS_TILE_TRACE): the caller's device
    // buffer, its size and the words handed out so far
    uint64_t *trace = nullptr;
    uint64_t trace_words = 0;
    uint64_t trace_used = 0;
};

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


// ------------------------------------------- scratch of the no-alloc entry

// Device memory that radix_sort_pairs_no_alloc uses as its workspace, so it
// needs no allocation.  Every GPU the library runs on holds its own copy for
// the life of the process.  Host code never uses the name itself (on the host
// it stands for a host-side symbol, not a device address): it uses the device
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[LRS_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices];  // per device; set once, under the mutex

// The current device's scratch address, looked up on the first call on each
// device (with that device current); NULL if the runtime cannot give it.
void *scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

namespace {

#ifndef LRS_MIN_TILES
#define LRS_MIN_TILES 256
#endif
// Fewest tiles a larger tile shape must still give: one per CU (4M keys take
// 512 8192-key tiles, 22% faster per sort than 1024 4096-key tiles).
constexpr uint64_t kMinTiles = LRS_MIN_TILES;
// Rows up to this length are sorted whole inside one workgroup's LDS.
constexpr uint64_t kResidentMax = 8192;
// Calls over at most this many elements are paced by the host: their timed
// launches are bracketed by recorded events (see TimedLaunch).
#ifndef LRS_HOST_PACED_MAX
#define LRS_HOST_PACED_MAX 65536
#endif
constexpr uint64_t kHostPacedMax = LRS_HOST_PACED_MAX;
// Longer index row sorts of rows up to this length carry each element as one
// 32-bit word, key << 16 | column, between passes.
constexpr uint64_t kPackedRowMax = 65536;

// The largest tile shape with at least kMinTiles tiles and at most 1/32 of
// its elements past row ends (rows of 65536 take eight 8192-key tiles, not
// five 15360-key tiles with 15% padding).
int choose_tile_cfg(uint64_t rows, uint64_t row_len, bool key64, bool keys_only) {
    for (int c = 2; c >= 1; --c) {
        const uint64_t tile = tile_cfg_of(key64, c, keys_only).tile;
        const uint64_t tiles = rows * ((row_len + tile - 1) / tile);
        const uint64_t padded = tiles * tile;
        if (tiles >= kMinTiles && (padded - rows * row_len) * 32 <= padded) return c;
    }
    return 0;
}
constexpr uint64_t kAlign = 256;
#ifndef LRS_HIST_BLOCKS
#define LRS_HIST_BLOCKS 256
#endif
// Histogram workgroups per launch: 1024 threads and 128 KB of LDS counters
// each, so one per CU at a time, and 256 of them fill the GPU once (one round
// of long spans; 512 and 1024 workgroups, two and four rounds, measured
// slower on 2^27 and 2^28 keys, as did smaller workgroups with fewer copies).
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

// ------------------------------------------------------------ per call

constexpr size_t kMaxTimed = 65536;

// Polls of an unpublished look-back word before a tile counts its prefix from
// the keys (about 1 us each, so the default is tens of milliseconds: far beyond
// any wait of a running sort, and only a guarantee against waiting forever).
constexpr uint32_t kDefaultSpinLimit = LRS_DEFAULT_SPIN_LIMIT;
// Partitions of the reduce-then-scan path: two workgroups per CU.
constexpr uint64_t kPartitions = 512;

// Everything one call needs besides its arguments: the stream and the
// caller's options.  Nothing is kept between calls.
struct Ctx {
    hipStream_t s = nullptr;
    lrs_timer *timer = nullptr;
    uint32_t spin_limit = kDefaultSpinLimit;  // 0: every tile counts its prefix from the keys
    int scan = LRS_SCAN_LOOKBACK;
    uint64_t wide_from = 0;
    uint64_t elems = ~uint64_t(0);  // elements the call handles (sets how a timer times it)
};

// False for an invalid option.
bool make_ctx(void *stream, const lrs_options *o, Ctx &c) {
    c.s = static_cast<hipStream_t>(stream);
    if (o == nullptr) return true;
    if (o->scan_strategy != LRS_SCAN_LOOKBACK && o->scan_strategy != LRS_SCAN_REDUCE_THEN_SCAN) return false;
    c.scan = o->scan_strategy;
    c.timer = o->timer;
    // Timer events are for calls run eagerly: a timed call on a stream being
    // captured into a graph is refused before anything is enqueued.
    if (c.timer != nullptr && c.s != nullptr) {
        hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(c.s, &st) != hipSuccess || st != hipStreamCaptureStatusNone) return false;
    }
    if (o->spin_limit != 0) c.spin_limit = o->spin_limit;
    if (o->prefix_from_keys) c.spin_limit = 0;
    c.wide_from = o->wide_from;
    return true;
}

uint64_t wide_from_of(const lrs_options *o) { return o ? o->wide_from : 0; }
bool options_ok(const lrs_options *o) {
    Ctx c;
    return make_ctx(nullptr, o, c);
}

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
    bool keys_only = false;         // sweeps with no payload phase (their own tile shapes)
    bool packed = false;            // row sort carrying key << 16 | column words between passes
    uint32_t hist_chunks_per_row = 0;
    // workspace layout (byte offsets)
    uint64_t off_hist = 0, hist_words = 0;
    uint64_t off_bases = 0;                      // hist_words bucket bases
    uint64_t off_counters = 0, counter_words = 0;  // finished histogram workgroups, per row
    uint64_t off_status[2] = {0, 0}, status_bytes = 0;
    uint64_t off_alt_keys = 0, off_alt_vals = 0, off_idx[2] = {0, 0};
    uint64_t total = 0;
};

// kind: 0 keys, 1 pairs, 2 segmented; key_bytes: 4 or 8 (segmented keys are 2 bytes)
// wide_from: nonzero sends rows of at least that many elements (sorted by
// sweeps) to the wide sweep as well.  row_index: a segmented sort whose
// payload is the column index the kernels make (not a caller's payload).
Plan make_plan(uint64_t rows, uint64_t row_len, int begin_bit, int end_bit, int b, int kind, int key_bytes = 4,
               uint64_t wide_from = 0, bool row_index = true) {
    Plan p;
    const bool key64 = key_bytes == 8;
    p.rows = rows;
    p.row_len = row_len;
    p.b = b;
    p.begin_bit = begin_bit;
    p.end_bit = end_bit;
    p.passes = static_cast<int>(cdiv(static_cast<uint64_t>(end_bit - begin_bit), b));
    const uint64_t R = 1ull << b;
    // A row needs the wide sweep (64-bit look-back words, 64-bit store
    // addresses) once its byte offsets pass what a 32-bit buffer offset
    // reaches (2^32 bytes) or its counts pass the 30-bit count of a 32-bit
    // look-back word: from 2^30 elements of 4 bytes, and from 2^29 for 8-byte
    // keys and for row sorts (int64 index out).
    const uint64_t widest = (kind == 2) ? 8 : static_cast<uint64_t>(key_bytes);
    p.wide_status = row_len * widest >= (1ull << 32) || row_len >= (1ull << 30);
    const bool resident = row_len <= kResidentMax && !key64;
    if (wide_from != 0 && row_len >= wide_from && !resident) p.wide_status = true;
    p.packed = kind == 2 && row_index && row_len <= kPackedRowMax && !p.wide_status;
    p.keys_only = !key64 && (kind == 0 || p.packed);
    // the wide sweep exists for the largest tile shape only
    p.tile_cfg = p.wide_status ? 2 : choose_tile_cfg(rows, row_len, key64, p.keys_only);
    p.tiles_per_row = static_cast<uint32_t>(cdiv(row_len, tile_cfg_of(key64, p.tile_cfg, p.keys_only).tile));
    p.num_tiles = rows * p.tiles_per_row;

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
    p.off_bases = off;
    off = align_up(off + 4 * p.hist_words, kAlign);
    p.off_counters = off;
    p.counter_words = rows;
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
    if (resident) {
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

// One launch, timed into a timer slot when the call has a timer.  For calls
// over many elements the dispatch itself stamps the slot's events, so nothing
// is enqueued between dependent kernels.  Calls over at most kHostPacedMax
// elements, whose launches the host rather than the GPU paces, bracket each
// launch with recorded events instead, which cost the host less per launch;
// the closing event is recorded when the TimedLaunch goes out of scope, so
// its scope must end right after the launch.
struct TimedLaunch {
    Launch L;  // the stream, and the slot's events when the dispatch stamps them
    hipEvent_t after = nullptr;  // bracketing: recorded by done() or on scope exit
    TimedLaunch(const TimedLaunch &) = delete;
    TimedLaunch &operator=(const TimedLaunch &) = delete;
    explicit TimedLaunch(int kind, const Ctx &c) {
        L.s = c.s;
        lrs_timer *t = c.timer;
        if (t == nullptr || t->used >= kMaxTimed) return;
        const bool bracket = c.elems <= kHostPacedMax;
        const size_t i = t->used;
        if (t->pool.size() < 2 * (i + 1)) {
            // The events only time: without the system-scope fence a recorded
            // event would otherwise add (a cache write-back and invalidation).
            hipEvent_t a, b;
            if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return;
            if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
                (void)hipEventDestroy(a);
                return;
            }
            t->pool.push_back(a);
            t->pool.push_back(b);
        }
        if (bracket) {
            if (hipEventRecord(t->pool[2 * i], c.s) != hipSuccess) return;
            after = t->pool[2 * i + 1];
        } else {
            L.start = t->pool[2 * i];
            L.stop = t->pool[2 * i + 1];
        }
        t->kind.resize(i + 1);
        t->kind[i] = kind;
        t->used = i + 1;
    }
    void done() {
        if (after != nullptr) (void)hipEventRecord(after, L.s);
        after = nullptr;
    }
    ~TimedLaunch() { done(); }
};

// Whole-row resident sort, timed as kind 4.
template <int KK, int PK>
hipError_t resident(int b, const ResidentArgs &a, uint64_t rows, uint64_t row_len, const Ctx &c) {
    TimedLaunch t(4, c);
    const hipError_t e = launch_resident<KK, PK>(b, a, rows, row_len, t.L);
    t.done();
    return e;
}

hipError_t launch_clear(const Plan &p, uint8_t *ws, bool need_hist, const Ctx &c) {
    ClearArgs a{};
    a.p[0] = need_hist ? reinterpret_cast<uint32_t *>(ws + p.off_hist) : nullptr;
    a.words[0] = p.hist_words;
    a.p[1] = reinterpret_cast<uint32_t *>(ws + p.off_counters);
    a.words[1] = p.counter_words;
    a.p[2] = reinterpret_cast<uint32_t *>(ws + p.off_status[0]);
    a.words[2] = p.status_bytes / 4;
    const uint64_t words = std::max<uint64_t>(a.words[0] * need_hist, a.words[2]);
    const uint32_t blocks = static_cast<uint32_t>(std::min<uint64_t>(2048, std::max<uint64_t>(1, cdiv(words / 4, kBlock))));
    TimedLaunch t(0, c);
    launch_on(clear_kernel, dim3(blocks), dim3(kBlock), t.L, a);
    hipError_t e = hipGetLastError();
    return e;
}

// All passes' digit counts into `hist`; with `ws` also the bucket bases (the
// row's last histogram workgroup scans them), for the sweeps.
hipError_t launch_histogram(const Plan &p, const void *keys, uint32_t *hist, int kk, uint64_t flip, uint64_t flip_neg,
                            bool accumulate, uint8_t *ws, const Ctx &c) {
    HistArgs h{};
    h.keys = keys;
    h.hist = hist;
    h.bases = ws ? reinterpret_cast<uint32_t *>(ws + p.off_bases) : nullptr;
    h.done = ws ? reinterpret_cast<uint32_t *>(ws + p.off_counters) : nullptr;
    h.row_len = static_cast<uint32_t>(p.row_len);
    h.chunks_per_row = p.hist_chunks_per_row;
    h.passes = static_cast<uint32_t>(p.passes);
    h.begin_bit = static_cast<uint32_t>(p.begin_bit);
    h.end_bit = static_cast<uint32_t>(p.end_bit);
    h.flip = flip;
    h.flip_neg = flip_neg;
    h.atomic = accumulate ? 1u : 0u;
    if (!accumulate && ws != nullptr) {
        h.status0 = reinterpret_cast<uint32_t *>(ws + p.off_status[0]);
        h.status0_row_words = static_cast<uint32_t>(p.status_bytes / 4 / p.rows);
    }
    const uint32_t blocks = static_cast<uint32_t>(p.rows * p.hist_chunks_per_row);
    TimedLaunch t(1, c);
    hipError_t e = (kk == kKeyU32)   ? launch_hist<kKeyU32>(p.b, h, blocks, t.L)
                   : (kk == kKeyC32) ? launch_hist<kKeyC32>(p.b, h, blocks, t.L)
                   : (kk == kKeyX32) ? launch_hist<kKeyX32>(p.b, h, blocks, t.L)
                   : (kk == kKeyU64) ? launch_hist<kKeyU64>(p.b, h, blocks, t.L)
                   : (kk == kKeyX64) ? launch_hist<kKeyX64>(p.b, h, blocks, t.L)
                                     : launch_hist<kKeyF16>(p.b, h, blocks, t.L);
    return e;
}

// `traced`: a look-back sweep, which records its tiles' phases in builds
// with LRS_TILE_TRACE when the call's timer has a trace buffer with room.
SweepArgs pass_args(const Plan &p, uint8_t *ws, int pass, const Ctx &c, bool traced = true) {
    SweepArgs a{};
    if (LRS_TILE_TRACE && traced && c.timer != nullptr && c.timer->trace != nullptr) {
        const uint64_t need = p.num_tiles * static_cast<uint64_t>(kTraceWords);
        if (c.timer->trace_used + need <= c.timer->trace_words) {
            a.trace = c.timer->trace + c.timer->trace_used;
            c.timer->trace_used += need;
        }
    }
    const uint64_t R = 1ull << p.b;
    a.bases = reinterpret_cast<const uint32_t *>(ws + p.off_bases) + static_cast<uint64_t>(pass) * R;
    a.bases_row_stride = static_cast<uint32_t>(p.passes * R);
    a.status = ws + p.off_status[pass & 1];
    a.status_next = (pass + 1 < p.passes) ? ws + p.off_status[(pass + 1) & 1] : nullptr;
    a.row_len = static_cast<uint32_t>(p.row_len);
    a.tiles_per_row = p.tiles_per_row;
    a.num_tiles = static_cast<uint32_t>(p.num_tiles);
    const int shift = p.begin_bit + pass * p.b;
    const int width = std::min(p.b, p.end_bit - shift);
    a.shift = static_cast<uint32_t>(shift);
    a.digit_mask = (1u << width) - 1u;
    a.flip = 0;
    a.flip_neg = 0;
    a.spin_limit = c.spin_limit;
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
// complement it for descending order (see KeyTraits<kKeyX32>); where both masks
// are equal (signed integers, descending u32) the image is one XOR (kKeyC32).
bool key_transform(int key_type, int descending, int &kk, uint64_t &flip, uint64_t &flip_neg) {
    const uint64_t c = descending ? ~0ull : 0ull;
    const uint64_t c32 = c & 0xFFFFFFFFull;
    const uint64_t top64 = 1ull << 63;
    switch (key_type) {
        case LRS_KEY_U32: kk = descending ? kKeyC32 : kKeyU32; flip = c32; flip_neg = c32; return true;
        case LRS_KEY_I32: kk = kKeyC32; flip = 0x80000000ull ^ c32; flip_neg = 0x80000000ull ^ c32; return true;
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

// Every pass's digit counts and bucket bases, before the first pass.  With
// several histogram workgroups per row their counts meet in global atomics,
// so the histogram, the finished-workgroup counters and the first pass's
// look-back words are cleared by a launch of their own first; with one per
// row the histogram kernel stores the counts and clears the row's first-pass
// look-back words itself (one launch fewer).
hipError_t launch_counts(const Plan &p, const void *keys, uint32_t *hist, int kk, uint64_t flip, uint64_t flip_neg,
                         uint8_t *ws, const Ctx &c) {
    const bool accumulate = p.hist_chunks_per_row > 1;
    if (accumulate && launch_clear(p, ws, true, c) != hipSuccess) return hipErrorLaunchFailure;
    return launch_histogram(p, keys, hist, kk, flip, flip_neg, accumulate, ws, c);
}

// Reduce-then-scan passes (CUDA Handbook ch.16: count, scan the counts, scatter;
// 100 Days of GPU, Day 35: persistent blocks walking their tiles in order): per
// pass, an upsweep counts the digit over each of up to 512 partitions of whole
// tiles, one workgroup scans those counts into start offsets, and the sweep
// sorts each partition's tiles in order from them.  No histogram kernel, no
// look-back; the upsweep reads the keys once more per pass.
int sort_32_reduce_then_scan(const Plan &p, int kk, uint64_t flip, uint64_t flip_neg, bool pairs,
                             const uint32_t *keys_in, const uint32_t *vals_in, uint32_t *keys_out,
                             uint32_t *vals_out, uint8_t *ws, const Ctx &c) {
    const uint64_t part_tiles = cdiv(p.num_tiles, std::min<uint64_t>(p.num_tiles, kPartitions));
    const uint64_t partitions = cdiv(p.num_tiles, part_tiles);
    uint32_t *counts = reinterpret_cast<uint32_t *>(ws + p.off_status[0]);  // partitions x R <= tiles x R
    uint32_t *alt_k = reinterpret_cast<uint32_t *>(ws + p.off_alt_keys);
    uint32_t *alt_v = reinterpret_cast<uint32_t *>(ws + p.off_alt_vals);
    const uint32_t *src_k = keys_in;
    const uint32_t *src_v = vals_in;
    for (int pass = 0; pass < p.passes; ++pass) {
        SweepArgs a = pass_args(p, ws, pass, c, false);
        PartArgs pa{};
        pa.keys = src_k;
        pa.counts = counts;
        pa.n = static_cast<uint32_t>(p.row_len);
        pa.part_len = static_cast<uint32_t>(part_tiles * tile_cfg_of(false, p.tile_cfg, p.keys_only).tile);
        pa.partitions = static_cast<uint32_t>(partitions);
        pa.shift = a.shift;
        pa.digit_mask = a.digit_mask;
        pa.flip = flip;
        pa.flip_neg = flip_neg;
        {
            TimedLaunch t(1, c);
            const hipError_t e = (kk == kKeyU32)   ? launch_partition_counts<kKeyU32>(p.b, pa, t.L)
                                 : (kk == kKeyC32) ? launch_partition_counts<kKeyC32>(p.b, pa, t.L)
                                                   : launch_partition_counts<kKeyX32>(p.b, pa, t.L);
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
        TimedLaunch t(2, c);
        if (pairs) {
            uint32_t *dv = pass_dst(pass, p.passes, vals_out, alt_v);
            a.vals_in = src_v;
            a.vals_out = dv;
            e = (kk == kKeyU32)   ? launch_sweep<kKeyU32, kPayU32, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, t.L)
                : (kk == kKeyC32) ? launch_sweep<kKeyC32, kPayU32, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, t.L)
                                  : launch_sweep<kKeyX32, kPayU32, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, t.L);
            src_v = dv;
        } else {
            e = (kk == kKeyU32)   ? launch_sweep<kKeyU32, kPayNone, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, t.L)
                : (kk == kKeyC32) ? launch_sweep<kKeyC32, kPayNone, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, t.L)
                                  : launch_sweep<kKeyX32, kPayNone, true>(p.b, a, p.tile_cfg, p.wide_status, partitions, t.L);
        }
        if (e != hipSuccess) return LRS_ERR_HIP;
        src_k = dk;
    }
    return LRS_OK;
}

// Keys of 32 bits: u32 as they are (KK = kKeyU32), anything else through the
// two-mask transform (KK = kKeyX32) or one constant XOR (KK = kKeyC32).
int sort_32(int kk, uint64_t flip, uint64_t flip_neg, bool pairs, const uint32_t *keys_in,
            const uint32_t *vals_in, uint32_t *keys_out, uint32_t *vals_out, uint64_t n, int begin_bit,
            int end_bit, int b, void *workspace, size_t ws_bytes, void *stream, const lrs_options *opts) {
    Ctx c;
    if (!make_ctx(stream, opts, c)) return LRS_ERR_OPTION;
    c.elems = n;
    if (!digit_bits_ok(b)) return LRS_ERR_DIGIT_BITS;
    if (begin_bit < 0 || end_bit > 32 || begin_bit >= end_bit) return LRS_ERR_BIT_RANGE;
    if (n > LRS_MAX_KEYS) return LRS_ERR_SIZE;
    if (n == 0) return LRS_OK;
    const Plan p = make_plan(1, n, begin_bit, end_bit, b, pairs ? 1 : 0, 4, c.wide_from);
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
            e = pairs ? resident<kKeyU32, kResU32>(b, r, 1, n, c) : resident<kKeyU32, kResNone>(b, r, 1, n, c);
        else if (kk == kKeyC32)
            e = pairs ? resident<kKeyC32, kResU32>(b, r, 1, n, c) : resident<kKeyC32, kResNone>(b, r, 1, n, c);
        else
            e = pairs ? resident<kKeyX32, kResU32>(b, r, 1, n, c) : resident<kKeyX32, kResNone>(b, r, 1, n, c);
        return e == hipSuccess ? LRS_OK : LRS_ERR_HIP;
    }
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    if (c.scan == LRS_SCAN_REDUCE_THEN_SCAN)
        return sort_32_reduce_then_scan(p, kk, flip, flip_neg, pairs, keys_in, vals_in, keys_out, vals_out, ws, c);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + p.off_hist);
    if (launch_counts(p, keys_in, hist, kk, flip, flip_neg, ws, c) != hipSuccess) return LRS_ERR_HIP;

    uint32_t *alt_k = reinterpret_cast<uint32_t *>(ws + p.off_alt_keys);
    uint32_t *alt_v = reinterpret_cast<uint32_t *>(ws + p.off_alt_vals);
    const uint32_t *src_k = keys_in;
    const uint32_t *src_v = vals_in;
    for (int pass = 0; pass < p.passes; ++pass) {
        SweepArgs a = pass_args(p, ws, pass, c);
        uint32_t *dk = pass_dst(pass, p.passes, keys_out, alt_k);
        a.keys_in = src_k;
        a.keys_out = dk;
        a.flip = flip;
        a.flip_neg = flip_neg;
        hipError_t e;
        TimedLaunch t(2, c);
        if (pairs) {
            uint32_t *dv = pass_dst(pass, p.passes, vals_out, alt_v);
            a.vals_in = src_v;
            a.vals_out = dv;
            e = (kk == kKeyU32)   ? launch_sweep<kKeyU32, kPayU32, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L)
                : (kk == kKeyC32) ? launch_sweep<kKeyC32, kPayU32, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L)
                                  : launch_sweep<kKeyX32, kPayU32, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L);
            src_v = dv;
        } else {
            e = (kk == kKeyU32)   ? launch_sweep<kKeyU32, kPayNone, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L)
                : (kk == kKeyC32) ? launch_sweep<kKeyC32, kPayNone, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L)
                                  : launch_sweep<kKeyX32, kPayNone, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L);
        }
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
            int end_bit, int b, void *workspace, size_t ws_bytes, void *stream, const lrs_options *opts) {
    Ctx c;
    if (!make_ctx(stream, opts, c)) return LRS_ERR_OPTION;
    c.elems = n;
    if (!digit_bits_ok(b)) return LRS_ERR_DIGIT_BITS;
    if (begin_bit < 0 || end_bit > 64 || begin_bit >= end_bit) return LRS_ERR_BIT_RANGE;
    if (n > LRS_MAX_KEYS) return LRS_ERR_SIZE;
    if (n == 0) return LRS_OK;
    const Plan p = make_plan(1, n, begin_bit, end_bit, b, pairs ? 1 : 0, 8, c.wide_from);
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

    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + p.off_hist);
    if (launch_counts(p, keys_in, hist, kk, flip, flip_neg, ws, c) != hipSuccess) return LRS_ERR_HIP;
    uint64_t *alt_k = reinterpret_cast<uint64_t *>(ws + p.off_alt_keys);
    uint32_t *alt_v = reinterpret_cast<uint32_t *>(ws + p.off_alt_vals);
    const uint64_t *src_k = keys_in;
    const uint32_t *src_v = vals_in;
    for (int pass = 0; pass < p.passes; ++pass) {
        SweepArgs a = pass_args(p, ws, pass, c);
        uint64_t *dk = pass_dst(pass, p.passes, keys_out, alt_k);
        a.keys_in = src_k;
        a.keys_out = dk;
        a.flip = flip;
        a.flip_neg = flip_neg;
        hipError_t e;
        TimedLaunch t(2, c);
        if (pairs) {
            uint32_t *dv = pass_dst(pass, p.passes, vals_out, alt_v);
            a.vals_in = src_v;
            a.vals_out = dv;
            e = (kk == kKeyU64) ? launch_sweep<kKeyU64, kPayU32, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L)
                                : launch_sweep<kKeyX64, kPayU32, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L);
            src_v = dv;
        } else {
            e = (kk == kKeyU64) ? launch_sweep<kKeyU64, kPayNone, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L)
                                : launch_sweep<kKeyX64, kPayNone, false>(b, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L);
        }
        if (e != hipSuccess) return LRS_ERR_HIP;
        src_k = dk;
    }
    return LRS_OK;
}

// Shape checks shared by the two row sorts; LRS_OK or the status to return.
int check_rows(int64_t rows, int64_t n, int dtype, int digit_bits) {
    if (!digit_bits_ok(digit_bits)) return LRS_ERR_DIGIT_BITS;
    if (dtype != LRS_DTYPE_FP16 && dtype != LRS_DTYPE_BF16) return LRS_ERR_DTYPE;
    if (rows < 0 || n < 0 || static_cast<uint64_t>(n) > LRS_MAX_ROW_LEN ||
        (rows > 0 && static_cast<uint64_t>(rows) * static_cast<uint64_t>(n) >= (1ull << 40)))
        return LRS_ERR_SIZE;
    return LRS_OK;
}

// Row sorts: rows x n 16-bit patterns; payload either the column index made in
// the kernels (pay_in == NULL, idx_out int64) or a caller's u32 per element.
int row_sort(const uint16_t *vals_in, const uint32_t *pay_in, uint16_t *vals_out, void *pay_out, int64_t rows,
             int64_t n, int dtype, int descending, int digit_bits, void *workspace, size_t workspace_bytes,
             void *stream, const lrs_options *opts) {
    Ctx c;
    if (!make_ctx(stream, opts, c)) return LRS_ERR_OPTION;
    c.elems = static_cast<uint64_t>(rows < 0 ? 0 : rows) * static_cast<uint64_t>(n < 0 ? 0 : n);
    const int st = check_rows(rows, n, dtype, digit_bits);
    if (st != LRS_OK) return st;
    if (rows == 0 || n == 0) return LRS_OK;
    const bool index = pay_in == nullptr;
    const Plan p = make_plan(rows, n, 0, 16, digit_bits, 2, 4, c.wide_from, index);
    if (!vals_in || !vals_out || !pay_out || (p.total && !workspace)) return LRS_ERR_NULL_POINTER;
    const uint64_t pay_size = index ? 8 : 4;
    if (misaligned(vals_in, 2) || misaligned(vals_out, 2) || misaligned(pay_out, pay_size) ||
        (!index && misaligned(pay_in, 4)) || misaligned(workspace, 256))
        return LRS_ERR_ALIGNMENT;
    if (p.num_tiles > 0x7FFFFFFFull || p.rows * p.hist_chunks_per_row > 0x7FFFFFFFull) return LRS_ERR_SIZE;
    if (p.resident && rows > 0x7FFFFFFF) return LRS_ERR_SIZE;
    if (workspace_bytes < p.total) return LRS_ERR_WORKSPACE_TOO_SMALL;
    const uint64_t cnt = static_cast<uint64_t>(rows) * n;
    const uint64_t vb = 2 * cnt, pb = pay_size * cnt, ib = 4 * cnt;
    if (overlaps(vals_out, vb, vals_in, vb) || overlaps(pay_out, pb, vals_in, vb) ||
        overlaps(pay_out, pb, vals_out, vb) || overlaps(vals_out, vb, workspace, p.total) ||
        overlaps(pay_out, pb, workspace, p.total) ||
        (!index && (overlaps(vals_out, vb, pay_in, ib) || overlaps(pay_out, pb, pay_in, ib))))
        return LRS_ERR_ALIASING;

    const uint32_t flip = descending ? 0xFFFFu : 0u;
    if (p.resident) {
        RowResidentArgs r{};
        r.keys_in = vals_in;
        r.keys_out = vals_out;
        r.pay_in = pay_in;
        r.pay_out = pay_out;
        r.rows = static_cast<uint32_t>(rows);
        r.row_len = static_cast<uint32_t>(n);
        r.flip = flip;
        TimedLaunch t(4, c);
        const hipError_t e = index ? launch_row_resident<kResIndex>(digit_bits, r, t.L)
                                   : launch_row_resident<kResU32>(digit_bits, r, t.L);
        t.done();
        return e == hipSuccess ? LRS_OK : LRS_ERR_HIP;
    }
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + p.off_hist);
    if (launch_counts(p, vals_in, hist, kKeyF16, flip, 0, ws, c) != hipSuccess) return LRS_ERR_HIP;

    uint16_t *alt_k = reinterpret_cast<uint16_t *>(ws + p.off_alt_keys);
    uint32_t *idx[2] = {reinterpret_cast<uint32_t *>(ws + p.off_idx[0]),
                        reinterpret_cast<uint32_t *>(ws + p.off_idx[1])};
    if (p.packed) {
        // Key and column travel as one word, key << 16 | column: the first
        // pass makes the words, the middle passes sort them by their high
        // half, the last pass writes the patterns and int64 columns back.
        // Each element moves 4 bytes between passes instead of 2 + 4, and no
        // pass but the last has a separate payload phase.
        const uint32_t *src_w = nullptr;
        for (int pass = 0; pass < p.passes; ++pass) {
            SweepArgs a = pass_args(p, ws, pass, c);
            a.flip = flip;
            uint32_t *dw = idx[pass & 1];
            hipError_t e;
            TimedLaunch t(2, c);
            if (pass == 0) {
                a.keys_in = vals_in;
                a.keys_out = dw;
                e = launch_sweep<kKeyF16, kPayPackFirst, false>(digit_bits, a, p.tile_cfg, false, p.num_tiles, t.L);
            } else {
                // the words' digit fields sit 16 bits above the key's
                a.shift += 16;
                a.keys_in = src_w;
                const bool last = pass + 1 == p.passes;
                a.keys_out = last ? static_cast<void *>(vals_out) : static_cast<void *>(dw);
                a.vals_out = last ? pay_out : nullptr;
                e = last ? launch_sweep<kKeyU32, kPayUnpackLast, false>(digit_bits, a, p.tile_cfg, false, p.num_tiles, t.L)
                         : launch_sweep<kKeyU32, kPayNone, false>(digit_bits, a, p.tile_cfg, false, p.num_tiles, t.L);
            }
            if (e != hipSuccess) return LRS_ERR_HIP;
            src_w = dw;
        }
        return LRS_OK;
    }
    const uint16_t *src_k = vals_in;
    const uint32_t *src_p = pay_in;
    for (int pass = 0; pass < p.passes; ++pass) {
        SweepArgs a = pass_args(p, ws, pass, c);
        a.flip = flip;
        uint16_t *dk = pass_dst(pass, p.passes, vals_out, alt_k);
        a.keys_in = src_k;
        a.keys_out = dk;
        hipError_t e;
        TimedLaunch t(2, c);
        if (!index) {
            // the caller's payload ping-pongs between pay_out and the first index buffer
            uint32_t *dp = pass_dst(pass, p.passes, static_cast<uint32_t *>(pay_out), idx[0]);
            a.vals_in = src_p;
            a.vals_out = dp;
            e = launch_sweep<kKeyF16, kPayU32, false>(digit_bits, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L);
            src_p = dp;
        } else if (pass == 0) {
            a.vals_in = nullptr;
            a.vals_out = idx[0];
            e = launch_sweep<kKeyF16, kPayIdxFirst, false>(digit_bits, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L);
        } else if (pass + 1 < p.passes) {
            a.vals_in = idx[(pass - 1) & 1];
            a.vals_out = idx[pass & 1];
            e = launch_sweep<kKeyF16, kPayU32, false>(digit_bits, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L);
        } else {
            a.vals_in = idx[(pass - 1) & 1];
            a.vals_out = pay_out;
            e = launch_sweep<kKeyF16, kPayIdxLast, false>(digit_bits, a, p.tile_cfg, p.wide_status, p.num_tiles, t.L);
        }
        if (e != hipSuccess) return LRS_ERR_HIP;
        src_k = dk;
    }
    return LRS_OK;
}

}  // namespace
}  // namespace lrs

using namespace lrs;

extern "C" {

size_t radix_sort_workspace_size(uint64_t n, int begin_bit, int end_bit, int digit_bits, int with_values,
                                 const lrs_options *opts) {
    if (!options_ok(opts) || !digit_bits_ok(digit_bits) || begin_bit < 0 || end_bit > 32 || begin_bit >= end_bit ||
        n == 0 || n > LRS_MAX_KEYS)
        return 0;
    return static_cast<size_t>(
        make_plan(1, n, begin_bit, end_bit, digit_bits, with_values ? 1 : 0, 4, wide_from_of(opts)).total);
}

int radix_sort_keys(const uint32_t *keys_in, uint32_t *keys_out, uint64_t n, int begin_bit, int end_bit,
                    int digit_bits, void *workspace, size_t workspace_bytes, void *stream, const lrs_options *opts) {
    return sort_32(kKeyU32, 0, 0, false, keys_in, nullptr, keys_out, nullptr, n, begin_bit, end_bit, digit_bits,
                   workspace, workspace_bytes, stream, opts);
}

int radix_sort_pairs(const uint32_t *keys_in, const uint32_t *vals_in, uint32_t *keys_out, uint32_t *vals_out,
                     uint64_t n, int begin_bit, int end_bit, int digit_bits, void *workspace, size_t workspace_bytes,
                     void *stream, const lrs_options *opts) {
    return sort_32(kKeyU32, 0, 0, true, keys_in, vals_in, keys_out, vals_out, n, begin_bit, end_bit, digit_bits,
                   workspace, workspace_bytes, stream, opts);
}

size_t radix_sort_typed_workspace_size(uint64_t n, int key_type, int begin_bit, int end_bit, int digit_bits,
                                       int with_values, const lrs_options *opts) {
    int kk;
    uint64_t flip, flip_neg;
    if (!options_ok(opts) || !key_transform(key_type, 0, kk, flip, flip_neg)) return 0;
    const int key_bits = key_type_is_64(key_type) ? 64 : 32;
    if (!digit_bits_ok(digit_bits) || begin_bit < 0 || end_bit > key_bits || begin_bit >= end_bit || n == 0 ||
        n > LRS_MAX_KEYS)
        return 0;
    return static_cast<size_t>(make_plan(1, n, begin_bit, end_bit, digit_bits, with_values ? 1 : 0, key_bits / 8,
                                         wide_from_of(opts)).total);
}

int radix_sort_keys_typed(const void *keys_in, void *keys_out, uint64_t n, int key_type, int descending,
                          int begin_bit, int end_bit, int digit_bits, void *workspace, size_t workspace_bytes,
                          void *stream, const lrs_options *opts) {
    int kk;
    uint64_t flip, flip_neg;
    if (!key_transform(key_type, descending, kk, flip, flip_neg)) return LRS_ERR_DTYPE;
    if (key_type_is_64(key_type))
        return sort_64(kk, flip, flip_neg, false, static_cast<const uint64_t *>(keys_in), nullptr,
                       static_cast<uint64_t *>(keys_out), nullptr, n, begin_bit, end_bit, digit_bits, workspace,
                       workspace_bytes, stream, opts);
    return sort_32(kk, flip, flip_neg, false, static_cast<const uint32_t *>(keys_in), nullptr,
                   static_cast<uint32_t *>(keys_out), nullptr, n, begin_bit, end_bit, digit_bits, workspace,
                   workspace_bytes, stream, opts);
}

int radix_sort_pairs_typed(const void *keys_in, const uint32_t *vals_in, void *keys_out, uint32_t *vals_out,
                           uint64_t n, int key_type, int descending, int begin_bit, int end_bit, int digit_bits,
                           void *workspace, size_t workspace_bytes, void *stream, const lrs_options *opts) {
    int kk;
    uint64_t flip, flip_neg;
    if (!key_transform(key_type, descending, kk, flip, flip_neg)) return LRS_ERR_DTYPE;
    if (key_type_is_64(key_type))
        return sort_64(kk, flip, flip_neg, true, static_cast<const uint64_t *>(keys_in), vals_in,
                       static_cast<uint64_t *>(keys_out), vals_out, n, begin_bit, end_bit, digit_bits, workspace,
                       workspace_bytes, stream, opts);
    return sort_32(kk, flip, flip_neg, true, static_cast<const uint32_t *>(keys_in), vals_in,
                   static_cast<uint32_t *>(keys_out), vals_out, n, begin_bit, end_bit, digit_bits, workspace,
                   workspace_bytes, stream, opts);
}

size_t segmented_row_sort_workspace_size(int64_t rows, int64_t n, int digit_bits, const lrs_options *opts) {
    if (!options_ok(opts) || check_rows(rows, n, LRS_DTYPE_FP16, digit_bits) != LRS_OK || rows == 0 || n == 0)
        return 0;
    // one size for both row sorts (index or caller payload)
    return static_cast<size_t>(std::max(make_plan(rows, n, 0, 16, digit_bits, 2, 4, wide_from_of(opts), true).total,
                                        make_plan(rows, n, 0, 16, digit_bits, 2, 4, wide_from_of(opts), false).total));
}

int segmented_row_sort(const uint16_t *vals_in, uint16_t *vals_out, int64_t *idx_out, int64_t rows, int64_t n,
                       int dtype, int descending, int digit_bits, void *workspace, size_t workspace_bytes,
                       void *stream, const lrs_options *opts) {
    return row_sort(vals_in, nullptr, vals_out, idx_out, rows, n, dtype, descending, digit_bits, workspace,
                    workspace_bytes, stream, opts);
}

int segmented_row_sort_pairs(const uint16_t *vals_in, const uint32_t *pay_in, uint16_t *vals_out,
                             uint32_t *pay_out, int64_t rows, int64_t n, int dtype, int descending,
                             int digit_bits, void *workspace, size_t workspace_bytes, void *stream,
                             const lrs_options *opts) {
    if (rows > 0 && n > 0 && pay_in == nullptr) return LRS_ERR_NULL_POINTER;
    return row_sort(vals_in, pay_in, vals_out, pay_out, rows, n, dtype, descending, digit_bits, workspace,
                    workspace_bytes, stream, opts);
}

int radix_sort_digit_histograms(const uint32_t *keys, uint64_t n, int begin_bit, int end_bit, int digit_bits,
                                uint32_t *hist_out, void *stream, const lrs_options *opts) {
    Ctx c;
    if (!make_ctx(stream, opts, c)) return LRS_ERR_OPTION;
    c.elems = n;
    if (!digit_bits_ok(digit_bits)) return LRS_ERR_DIGIT_BITS;
    if (begin_bit < 0 || end_bit > 32 || begin_bit >= end_bit) return LRS_ERR_BIT_RANGE;
    if (n > LRS_MAX_KEYS) return LRS_ERR_SIZE;
    if (!hist_out || (n && !keys)) return LRS_ERR_NULL_POINTER;
    if (misaligned(keys, 4) || misaligned(hist_out, 16)) return LRS_ERR_ALIGNMENT;
    const Plan p = make_plan(1, n ? n : 1, begin_bit, end_bit, digit_bits, 0);
    ClearArgs a{};
    a.p[0] = hist_out;
    a.words[0] = p.hist_words;
    {
        TimedLaunch t(0, c);
        launch_on(clear_kernel, dim3(1), dim3(kBlock), t.L, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return LRS_ERR_HIP;
    }
    if (n == 0) return LRS_OK;
    return launch_histogram(p, keys, hist_out, kKeyU32, 0, 0, true, nullptr, c) == hipSuccess ? LRS_OK : LRS_ERR_HIP;
}

int radix_sort_copy_probe(const void *src, void *dst, size_t bytes, void *stream, const lrs_options *opts) {
    Ctx c;
    if (!make_ctx(stream, opts, c)) return LRS_ERR_OPTION;
    c.elems = bytes / 4;
    if (bytes == 0) return LRS_OK;
    if (!src || !dst) return LRS_ERR_NULL_POINTER;
    if (misaligned(src, 16) || misaligned(dst, 16)) return LRS_ERR_ALIGNMENT;
    if (overlaps(src, bytes, dst, bytes)) return LRS_ERR_ALIASING;
    const uint64_t n16 = bytes / 16;
    const uint32_t tail = static_cast<uint32_t>(bytes % 16);
    const uint32_t blocks = static_cast<uint32_t>(std::min<uint64_t>(1u << 20, std::max<uint64_t>(1, cdiv(n16, kBlock))));
    TimedLaunch t(3, c);
    launch_on(copy_kernel, dim3(blocks), dim3(kBlock), t.L, static_cast<const uint4 *>(src), static_cast<uint4 *>(dst),
              n16, static_cast<const uint8_t *>(src) + n16 * 16, static_cast<uint8_t *>(dst) + n16 * 16, tail);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? LRS_OK : LRS_ERR_HIP;
}

int radix_sort_pairs_no_alloc(const uint32_t *keys_in, const uint32_t *vals_in, uint32_t *keys_out,
                              uint32_t *vals_out, uint64_t n, int begin_bit, int end_bit, int digit_bits, void *stream,
                              const lrs_options *opts) {
    if (!options_ok(opts)) return LRS_ERR_OPTION;
    if (!digit_bits_ok(digit_bits)) return LRS_ERR_DIGIT_BITS;
    if (begin_bit < 0 || end_bit > 32 || begin_bit >= end_bit) return LRS_ERR_BIT_RANGE;
    if (n == 0) return LRS_OK;
    if (n > LRS_MAX_KEYS) return LRS_ERR_SIZE;
    const uint64_t need = make_plan(1, n, begin_bit, end_bit, digit_bits, 1, 4, wide_from_of(opts)).total;
    if (need > LRS_NO_ALLOC_SCRATCH_BYTES) return LRS_ERR_SIZE;
    void *ws = nullptr;
    if (need > 0) {
        ws = scratch_address();
        if (ws == nullptr) return LRS_ERR_HIP;
    }
    return sort_32(kKeyU32, 0, 0, true, keys_in, vals_in, keys_out, vals_out, n, begin_bit, end_bit, digit_bits, ws,
                   LRS_NO_ALLOC_SCRATCH_BYTES, stream, opts);
}

lrs_timer *radix_sort_timer_create(void) {
    try {
        return new lrs_timer();
    } catch (...) {
        return nullptr;
    }
}

int radix_sort_timer_read(lrs_timer *timer, double *ms_by_kind, int *launches_by_kind) {
    for (int k = 0; k < 5; ++k) {
        if (ms_by_kind) ms_by_kind[k] = 0.0;
        if (launches_by_kind) launches_by_kind[k] = 0;
    }
    if (timer == nullptr) return LRS_ERR_NULL_POINTER;
    const size_t used = timer->used;
    timer->used = 0;
    for (size_t i = 0; i < used; ++i) {
        if (hipEventSynchronize(timer->pool[2 * i + 1]) != hipSuccess) return LRS_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, timer->pool[2 * i], timer->pool[2 * i + 1]) != hipSuccess) return LRS_ERR_HIP;
        const int k = timer->kind[i];
        if (ms_by_kind) ms_by_kind[k] += ms;
        if (launches_by_kind) launches_by_kind[k] += 1;
    }
    return LRS_OK;
}

static_assert(lrs::kTraceWords == LRS_TILE_TRACE_WORDS, "trace record size as declared");

int radix_sort_timer_trace_tiles(lrs_timer *timer, uint64_t *buf, uint64_t words) {
    if (timer == nullptr) return LRS_ERR_NULL_POINTER;
    if (!LRS_TILE_TRACE) return LRS_ERR_OPTION;  // a build without the records
    if (buf == nullptr && words != 0) return LRS_ERR_NULL_POINTER;
    if (misaligned(buf, 8)) return LRS_ERR_ALIGNMENT;
    timer->trace = buf;
    timer->trace_words = buf != nullptr ? words : 0;
    timer->trace_used = 0;
    return LRS_OK;
}

int radix_sort_timer_trace_used(const lrs_timer *timer, uint64_t *words) {
    if (timer == nullptr || words == nullptr) return LRS_ERR_NULL_POINTER;
    *words = timer->trace_used;
    return LRS_OK;
}

void radix_sort_timer_destroy(lrs_timer *timer) {
    if (timer == nullptr) return;
    for (hipEvent_t e : timer->pool) (void)hipEventDestroy(e);
    delete timer;
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
        case LRS_ERR_OPTION: return "an lrs_options field has an invalid value";
        default: return "unknown status";
    }
}

}  // extern "C"
