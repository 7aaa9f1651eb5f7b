// lrs_kernels.h -- gfx950 device code of the LSD radix sort (internal header,
// included by lrs_host.hip only).
//
// One pass of the sort is one launch of `sweep_kernel`: every workgroup takes
// the next tile of TILE keys in input order, ranks each key stably inside the
// tile by its digit, learns how many keys of each digit all earlier tiles of
// its row hold through a decoupled look-back over per-tile digit counts, and
// writes its keys (and payload) to  bucket base + earlier tiles' count + rank.
// The bucket bases come from `histogram_kernel`, which counts the digits of
// every pass in one read of the keys before the first pass.
//
// Pages this follows: CUDA Handbook ch.16 "Radix Sort" (histogram, exclusive
// scan, stable scatter; the GPU sample's per-tile histograms scanned
// digit-major, its local sort and its scatter by digit-run start); 100 Days of
// GPU, Day 35 (one-bit split, per-block histograms, the tile walk); FlagTree
// PR #1084 (all-pass histogram, tile offsets, compact int32 index payload with
// int64 only in the final pass, row-major tile order); gpu.rocks "The Whole
// Sort" (destination = bucket start + number of earlier same-digit keys).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrs {

constexpr int kBlock = 256;            // threads per workgroup
constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kWaves = kBlock / kWave;

enum KeyKind : int { kKeyU32 = 0, kKeyF16 = 1 };

// Payload handling of one pass.
enum PayKind : int {
    kPayNone = 0,      // keys only
    kPayU32 = 1,       // read u32, write u32 (pairs; middle passes of the row sort)
    kPayIdxFirst = 2,  // synthesise the column index, write u32 (first row-sort pass)
    kPayIdxLast = 3,   // read u32 index, write int64 (last row-sort pass)
};

// ------------------------------------------------------------- key traits

template <int KK> struct KeyTraits;

template <> struct KeyTraits<kKeyU32> {
    using Stored = uint32_t;
    // The sort key of a stored u32 is the value itself.
    __device__ static inline uint32_t key(uint32_t v, uint32_t) { return v; }
};

template <> struct KeyTraits<kKeyF16> {
    using Stored = uint16_t;
    // Order-preserving key of a 16-bit float pattern: complement negatives,
    // set the sign bit of non-negatives; `flip` = 0xFFFF complements the result
    // for descending order.
    __device__ static inline uint32_t key(uint32_t v, uint32_t flip) {
        uint32_t asc = v ^ ((v & 0x8000u) ? 0xFFFFu : 0x8000u);
        return asc ^ flip;
    }
};

// --------------------------------------------------------- wave utilities

// Lanes of this wave whose digit equals this lane's digit (all 64 lanes must
// be active): the AND, over the digit's B bits, of each bit's ballot or its
// complement.
template <int B>
__device__ inline uint64_t match_mask(uint32_t d) {
    uint64_t m = ~0ull;
#pragma unroll
    for (int i = 0; i < B; ++i) {
        const bool bit = (d >> i) & 1u;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

// Number of set bits of m at lanes below this lane.
__device__ inline uint32_t count_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ inline uint32_t wave_inclusive_scan(uint32_t x, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    return x;
}

// Workgroup-wide exclusive scan of one value per thread.  Every thread of the
// workgroup must call it.  `tmp` holds kWaves words of LDS.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t *tmp, int lane, int wave) {
    const uint32_t inc = wave_inclusive_scan(v, lane);
    if (lane == kWave - 1) tmp[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
        if (w < wave) before += tmp[w];
    __syncthreads();
    return before + inc - v;
}

// ------------------------------------------------------- look-back status

// One status word per (tile, digit): a 2-bit flag over the count.  Flag 0 =
// not yet published, 1 = this tile's own count, 2 = inclusive count of all
// tiles of the row up to and including this one.
template <typename W> struct Status {
    static constexpr int kShift = sizeof(W) * 8 - 2;
    static constexpr W kMask = (W(1) << kShift) - W(1);
    static constexpr W kAggregate = W(1) << kShift;
    static constexpr W kInclusive = W(2) << kShift;
};

template <typename W>
__device__ inline void publish(W *p, W v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename W>
__device__ inline W observe(const W *p) {
    return __hip_atomic_load(const_cast<W *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ sweep pass

struct SweepArgs {
    const void *keys_in;
    void *keys_out;
    const void *vals_in;
    void *vals_out;
    const uint32_t *hist;    // this pass's digit counts of row 0; row r at hist + r * hist_row_stride
    void *status;            // [num_tiles][R] look-back words of this pass
    void *status_next;       // the next pass's words, cleared here (NULL on the last pass)
    uint32_t *tile_counter;  // this pass's tile ticket counter, zero on entry
    uint32_t row_len;        // elements per row
    uint32_t tiles_per_row;
    uint32_t num_tiles;      // rows * tiles_per_row = grid size
    uint32_t hist_row_stride;
    uint32_t shift;          // lowest bit of this pass's digit
    uint32_t digit_mask;     // (1 << width) - 1
    uint32_t flip;           // 0xFFFF for descending 16-bit float keys, else 0
};

// How a wave finds the lanes that share its digit.
enum MatchKind : int { kMatchBallot = 0, kMatchLds = 1 };

template <int B, int ITEMS, int KK, int PK, typename W, int MATCH>
__global__ __launch_bounds__(kBlock) void sweep_kernel(SweepArgs a) {
    constexpr uint32_t R = 1u << B;
    constexpr uint32_t TILE = kBlock * ITEMS;
    using Stored = typename KeyTraits<KK>::Stored;
    using St = Status<W>;

    __shared__ uint32_t s_buf[TILE];          // tile in digit order: keys, then payload
    __shared__ uint32_t s_cnt[kWaves][R];     // per-wave digit counts, then per-wave bases
    __shared__ uint32_t s_goff[R];            // output index of digit run start minus local start
    __shared__ uint32_t s_tmp[kWaves];
    __shared__ uint32_t s_ticket;
    __shared__ unsigned long long s_match[MATCH == kMatchLds ? kWaves : 1][MATCH == kMatchLds ? R : 1];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    for (uint32_t i = tid; i < kWaves * R; i += kBlock) (&s_cnt[0][0])[i] = 0u;
    if constexpr (MATCH == kMatchLds)
        for (uint32_t i = tid; i < kWaves * R; i += kBlock) (&s_match[0][0])[i] = 0ull;
    if (tid == 0) s_ticket = atomicAdd(a.tile_counter, 1u);
    __syncthreads();

    // Tiles are handed out in ticket order, so every tile this one waits for
    // below is already running.  Tiles are numbered row-major.
    const uint32_t t = s_ticket;
    if (t >= a.num_tiles) return;  // cannot happen with a zeroed counter and grid == num_tiles
    const uint32_t row = t / a.tiles_per_row;
    const uint32_t tile_in_row = t - row * a.tiles_per_row;
    const uint32_t tile_start = tile_in_row * TILE;
    const uint32_t valid = min(TILE, a.row_len - tile_start);
    const uint64_t row_base = static_cast<uint64_t>(row) * a.row_len;

    const Stored *kin = static_cast<const Stored *>(a.keys_in) + row_base + tile_start;
    const uint32_t wbase = static_cast<uint32_t>(wave) * kWave * ITEMS;

    // Wave-striped load: item j of lane l is tile element wbase + j*64 + l, so
    // (item, lane) order is input order inside each wave.
    uint32_t key[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t p = wbase + j * kWave + lane;
        key[j] = (p < valid) ? static_cast<uint32_t>(kin[p]) : 0u;
    }
    uint32_t val[ITEMS];
    if constexpr (PK == kPayU32 || PK == kPayIdxLast) {
        const uint32_t *vin = static_cast<const uint32_t *>(a.vals_in) + row_base + tile_start;
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t p = wbase + j * kWave + lane;
            val[j] = (p < valid) ? vin[p] : 0u;
        }
    }

    // Stable rank inside the wave.  For item j, the lanes holding the same
    // digit form a group (found by ballots, or by OR-ing each lane's bit into a
    // per-digit mask in LDS); a lane's rank is the wave's running count of the
    // digit plus the group members at lower lanes, and the group's lowest lane
    // advances the running count (and clears the mask).  Elements past the end
    // of the row take the largest digit; being last in input order they rank
    // after every real key of that digit and are never written.
    const uint64_t lane_bit = 1ull << lane;
    uint32_t rank[ITEMS];  // digit << 16 | rank within the wave's digit
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t p = wbase + j * kWave + lane;
        const uint32_t d = (p < valid)
            ? ((KeyTraits<KK>::key(key[j], a.flip) >> a.shift) & a.digit_mask) : (R - 1u);
        uint64_t m;
        if constexpr (MATCH == kMatchBallot) {
            m = match_mask<B>(d);
        } else {
            atomicOr(&s_match[wave][d], static_cast<unsigned long long>(lane_bit));
            m = s_match[wave][d];
        }
        const uint32_t below = count_below(m);
        const uint32_t before = s_cnt[wave][d];
        rank[j] = (d << 16) | (before + below);
        if (below == 0u) {
            s_cnt[wave][d] = before + static_cast<uint32_t>(__popcll(m));
            if constexpr (MATCH == kMatchLds) s_match[wave][d] = 0ull;
        }
    }
    __syncthreads();

    // Digit d is owned by thread d: the tile's count of d, the waves' bases,
    // and the row's bucket base (exclusive scan of the pass histogram).
    uint32_t count = 0u;
    if (tid < static_cast<int>(R)) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t c = s_cnt[w][tid];
            s_cnt[w][tid] = count;
            count += c;
        }
    }
    // Publish this tile's own counts as early as possible.  Padding elements
    // are not part of the count of the last digit.
    uint32_t real = count;
    if (tid == static_cast<int>(R) - 1) real -= TILE - valid;
    W *status = static_cast<W *>(a.status) + static_cast<uint64_t>(t) * R;
    if (tid < static_cast<int>(R))
        publish(status + tid, static_cast<W>((tile_in_row == 0 ? St::kInclusive : St::kAggregate) |
                                             static_cast<W>(real)));

    const uint32_t local_start = block_exclusive_scan(count, s_tmp, lane, wave);
    const uint32_t hcount = (tid < static_cast<int>(R)) ? a.hist[static_cast<uint64_t>(row) * a.hist_row_stride + tid] : 0u;
    const uint32_t bucket_base = block_exclusive_scan(hcount, s_tmp, lane, wave);
    if (tid < static_cast<int>(R)) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s_cnt[w][tid] += local_start;
    }
    __syncthreads();

    // Local reorder: each key goes to its slot in the tile's digit order.
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t d = rank[j] >> 16;
        const uint32_t slot = s_cnt[wave][d] + (rank[j] & 0xFFFFu);
        s_buf[slot] = key[j];
        rank[j] = slot;
    }

    // Decoupled look-back: the count of digit d in all earlier tiles of the row.
    if (tid < static_cast<int>(R)) {
        W excl = 0;
        if (tile_in_row != 0) {
            const W *look = static_cast<const W *>(a.status) + static_cast<uint64_t>(t - 1u) * R + tid;
            for (;;) {
                const W s = observe(look);
                const W flag = s & ~St::kMask;
                if (flag == 0) {
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                excl += s & St::kMask;
                if (flag == St::kInclusive) break;
                look -= R;
            }
            publish(status + tid, static_cast<W>(St::kInclusive | (excl + real)));
        }
        s_goff[tid] = bucket_base + static_cast<uint32_t>(excl) - local_start;
        if (a.status_next != nullptr)
            static_cast<W *>(a.status_next)[static_cast<uint64_t>(t) * R + tid] = 0;
    }
    __syncthreads();

    // Write the keys: consecutive threads take consecutive slots, so each
    // digit run of the tile is written to consecutive addresses.
    Stored *kout = static_cast<Stored *>(a.keys_out) + row_base;
    uint32_t dst[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const uint32_t k = i * kBlock + tid;
        const uint32_t v = s_buf[k];
        const uint32_t d = (KeyTraits<KK>::key(v, a.flip) >> a.shift) & a.digit_mask;
        dst[i] = s_goff[d] + k;
        // dst < row_len holds for every real element; the test only keeps a
        // logic error from turning into a stray store
        if (k < valid && dst[i] < a.row_len) kout[dst[i]] = static_cast<Stored>(v);
    }

    if constexpr (PK != kPayNone) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            uint32_t v;
            if constexpr (PK == kPayIdxFirst) v = tile_start + wbase + j * kWave + lane;
            else v = val[j];
            s_buf[rank[j]] = v;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const uint32_t k = i * kBlock + tid;
            if (k < valid && dst[i] < a.row_len) {
                if constexpr (PK == kPayIdxLast)
                    static_cast<int64_t *>(a.vals_out)[row_base + dst[i]] = static_cast<int64_t>(s_buf[k]);
                else
                    static_cast<uint32_t *>(a.vals_out)[row_base + dst[i]] = s_buf[k];
            }
        }
    }
}

// ------------------------------------------------------- digit histograms

struct HistArgs {
    const void *keys;
    uint32_t *hist;          // [rows][passes][R], zero on entry when atomic != 0
    uint32_t row_len;
    uint32_t chunks_per_row;
    uint32_t chunk;          // elements per workgroup, a multiple of 8
    uint32_t passes;
    uint32_t begin_bit;
    uint32_t end_bit;
    uint32_t flip;
    uint32_t atomic;         // 1: several workgroups per row accumulate; 0: one writes it
};

constexpr int kHistMaxCounters = 1024;  // passes * R for every legal (window, b)

// Counts every pass's digit over one chunk of one row in LDS, from one read of
// the keys with 16-byte loads, then adds the counts to the row's histogram.
template <int B, int KK>
__global__ __launch_bounds__(kBlock) void histogram_kernel(HistArgs a) {
    constexpr uint32_t R = 1u << B;
    using Stored = typename KeyTraits<KK>::Stored;
    constexpr uint32_t kPerVec = 16u / sizeof(Stored);
    __shared__ uint32_t s_h[kHistMaxCounters];

    const uint32_t row = blockIdx.x / a.chunks_per_row;
    const uint32_t chunk = blockIdx.x - row * a.chunks_per_row;
    const uint32_t total = a.passes * R;
    for (uint32_t i = threadIdx.x; i < total; i += kBlock) s_h[i] = 0u;
    __syncthreads();

    const uint32_t lo = chunk * a.chunk;
    const uint32_t hi = min(a.row_len, lo + a.chunk);
    const Stored *base = static_cast<const Stored *>(a.keys) + static_cast<uint64_t>(row) * a.row_len;

    auto count_key = [&](uint32_t v) {
        const uint32_t k = KeyTraits<KK>::key(v, a.flip);
        for (uint32_t p = 0; p < a.passes; ++p) {
            const uint32_t shift = a.begin_bit + p * B;
            const uint32_t width = min(static_cast<uint32_t>(B), a.end_bit - shift);
            const uint32_t d = (k >> shift) & ((1u << width) - 1u);
            atomicAdd(&s_h[p * R + d], 1u);
        }
    };

    // 16-byte loads when the chunk starts 16-byte aligned; lo is a multiple of
    // the chunk size (a multiple of 8), so only the row start can misalign it.
    const uintptr_t addr = reinterpret_cast<uintptr_t>(base + lo);
    uint32_t i = lo;
    if ((addr & 15u) == 0u) {
        const uint32_t nvec = (hi - lo) / kPerVec;
        const uint4 *v4 = reinterpret_cast<const uint4 *>(base + lo);
        for (uint32_t q = threadIdx.x; q < nvec; q += kBlock) {
            const uint4 w = v4[q];
            if constexpr (KK == kKeyU32) {
                count_key(w.x); count_key(w.y); count_key(w.z); count_key(w.w);
            } else {
                count_key(w.x & 0xFFFFu); count_key(w.x >> 16);
                count_key(w.y & 0xFFFFu); count_key(w.y >> 16);
                count_key(w.z & 0xFFFFu); count_key(w.z >> 16);
                count_key(w.w & 0xFFFFu); count_key(w.w >> 16);
            }
        }
        i = lo + nvec * kPerVec;
    }
    for (uint32_t q = i + threadIdx.x; q < hi; q += kBlock) count_key(static_cast<uint32_t>(base[q]));
    __syncthreads();

    uint32_t *out = a.hist + static_cast<uint64_t>(row) * total;
    for (uint32_t q = threadIdx.x; q < total; q += kBlock) {
        const uint32_t c = s_h[q];
        if (a.atomic) {
            if (c) atomicAdd(out + q, c);
        } else {
            out[q] = c;
        }
    }
}

// ------------------------------------------------------- small utilities

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

__global__ __launch_bounds__(kBlock) void copy_kernel(const uint4 *src, uint4 *dst, uint64_t n16,
                                                      const uint8_t *src_tail, uint8_t *dst_tail,
                                                      uint32_t tail) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = blockIdx.x * static_cast<uint64_t>(kBlock) + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
    if (blockIdx.x == 0 && threadIdx.x < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

}  // namespace lrs
