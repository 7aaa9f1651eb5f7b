// lrs_kernels.h -- gfx950 device code of the LSD radix sort (internal header,
// included through lrs_launch.h; the lrs_inst_*.hip units compile it).
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

#include <type_traits>

namespace lrs {

// Compile-time tunables (defaults are the measured choices).
#ifndef LRS_SWEEP_ITEMS
#define LRS_SWEEP_ITEMS 30      // keys per thread in the largest sweep tile
#endif
#ifndef LRS_SWEEP_KEYS_ITEMS
#define LRS_SWEEP_KEYS_ITEMS 32 // the same for sweeps with no payload phase
#endif
#ifndef LRS_SWEEP_BLOCK
#define LRS_SWEEP_BLOCK 512     // threads per workgroup of the largest sweep tile
#endif
#ifndef LRS_LOOKBACK
#define LRS_LOOKBACK 4          // predecessor words a look-back lane reads per round trip
#endif
#ifndef LRS_HIST_COPIES
#define LRS_HIST_COPIES 32      // LDS copies of the histogram, lane l counts into copy l % 32
#endif
#ifndef LRS_XCD_CHUNK
#define LRS_XCD_CHUNK 16        // consecutive sweep tiles handed to one XCD at a time
#endif
#ifndef LRS_SWEEP_WAVES_PER_EU
#define LRS_SWEEP_WAVES_PER_EU 4  // register budget of the sweep (4: 128 VGPRs)
#endif
#ifndef LRS_PAYLOAD_EARLY
#define LRS_PAYLOAD_EARLY 2     // payload loads before the key write-out: 0 never, 1 always, 2 for 8-byte keys
#endif
#ifndef LRS_TILE_TRACE
#define LRS_TILE_TRACE 0        // measurement builds: look-back sweep tiles record their phase times
#endif
#ifndef LRS_RANK_PIPELINE
#define LRS_RANK_PIPELINE 1     // ballot rank builds item j+1's match mask while item j's counter read is in flight
#endif


constexpr int kBlock = 256;            // threads per workgroup (histogram, utilities)
constexpr int kSweepBlock = LRS_SWEEP_BLOCK;
constexpr int kLookback = LRS_LOOKBACK;
constexpr uint32_t kXcdChunk = LRS_XCD_CHUNK;
constexpr uint32_t kXcds = 8;          // accelerator complex dies (XCDs) of an MI355X
constexpr int kWave = 64;              // CDNA wavefront width

enum KeyKind : int { kKeyU32 = 0, kKeyF16 = 1, kKeyX32 = 2, kKeyU64 = 3, kKeyX64 = 4, kKeyC32 = 5 };

// Payload handling of one pass.
enum PayKind : int {
    kPayNone = 0,        // keys only
    kPayU32 = 1,         // read u32, write u32 (pairs; middle passes of the row sort)
    kPayIdxFirst = 2,    // synthesise the column index, write u32 (first row-sort pass)
    kPayIdxLast = 3,     // read u32 index, write int64 (last row-sort pass)
    // Row sorts of rows of at most 65536 elements carry key and column as one
    // word, key << 16 | column, between passes (the middle passes are
    // keys-only sorts of those words by their high half):
    kPayPackFirst = 4,   // 16-bit patterns in, words out (first pass)
    kPayUnpackLast = 5,  // words in; the pattern and its int64 column out (last pass)
};

// ------------------------------------------------------------- key traits

template <int KK> struct KeyTraits;

// key(v, flip, flip_neg) maps a stored pattern to the unsigned integer whose
// ascending order is the wanted order.  Word is the register type of a key
// (and of its slot in LDS); the masks are 64-bit, of which 16- and 32-bit keys
// use the low half.

template <> struct KeyTraits<kKeyU32> {
    using Stored = uint32_t;
    using Word = uint32_t;
    // The sort key of a stored u32 is the value itself.
    __device__ static inline uint32_t key(uint32_t v, uint64_t, uint64_t) { return v; }
};

template <> struct KeyTraits<kKeyF16> {
    using Stored = uint16_t;
    using Word = uint32_t;
    // Order-preserving key of a 16-bit float pattern: complement negatives,
    // set the sign bit of non-negatives; `flip` = 0xFFFF complements the result
    // for descending order.
    __device__ static inline uint32_t key(uint32_t v, uint64_t flip, uint64_t) {
        uint32_t asc = v ^ ((v & 0x8000u) ? 0xFFFFu : 0x8000u);
        return asc ^ static_cast<uint32_t>(flip);
    }
};

template <> struct KeyTraits<kKeyX32> {
    using Stored = uint32_t;
    using Word = uint32_t;
    // Any other 32-bit key: XOR with `flip` when the sign bit is clear and with
    // `flip_neg` when it is set.  Signed integers: both 0x80000000.  Floats:
    // 0x80000000 and 0xFFFFFFFF (set the sign bit of non-negatives, complement
    // negatives).  Descending order complements both masks (u32: both ~0).
    __device__ static inline uint32_t key(uint32_t v, uint64_t flip, uint64_t flip_neg) {
        return v ^ static_cast<uint32_t>((static_cast<int32_t>(v) < 0) ? flip_neg : flip);
    }
};

template <> struct KeyTraits<kKeyC32> {
    using Stored = uint32_t;
    using Word = uint32_t;
    // 32-bit keys whose order-preserving image is the pattern XORed with one
    // constant, whatever the sign bit: signed integers (0x80000000, and
    // 0x7FFFFFFF descending) and descending u32 (0xFFFFFFFF).  One XOR, where
    // kKeyX32's two masks take a compare and a select as well.
    __device__ static inline uint32_t key(uint32_t v, uint64_t flip, uint64_t) {
        return v ^ static_cast<uint32_t>(flip);
    }
};

template <> struct KeyTraits<kKeyU64> {
    using Stored = uint64_t;
    using Word = uint64_t;
    __device__ static inline uint64_t key(uint64_t v, uint64_t, uint64_t) { return v; }
};

template <> struct KeyTraits<kKeyX64> {
    using Stored = uint64_t;
    using Word = uint64_t;
    // As kKeyX32 with 64-bit masks (signed integers: both 2^63; doubles: 2^63
    // and ~0; complemented for descending order).
    __device__ static inline uint64_t key(uint64_t v, uint64_t flip, uint64_t flip_neg) {
        return v ^ ((static_cast<int64_t>(v) < 0) ? flip_neg : flip);
    }
};

// The pass digit of a key word: `mask` bits from bit `shift` of its key.
template <int KK>
__device__ inline uint32_t digit_of(typename KeyTraits<KK>::Word v, uint64_t flip, uint64_t flip_neg,
                                    uint32_t shift, uint32_t mask) {
    if constexpr (sizeof(typename KeyTraits<KK>::Word) == 8) {
        return static_cast<uint32_t>(KeyTraits<KK>::key(v, flip, flip_neg) >> shift) & mask;
    } else {
        // one bit-field extract (the width is uniform: a scalar popcount)
        return __builtin_amdgcn_ubfe(KeyTraits<KK>::key(v, flip, flip_neg), shift,
                                     static_cast<uint32_t>(__builtin_popcount(mask)));
    }
}

// Order-preserving key of a 16-bit float pattern and its inverse (negative
// patterns complemented, non-negative ones with the sign bit set; `flip`
// complements the key for descending order).
__device__ inline uint32_t f16_key(uint32_t v, uint32_t flip) {
    return (v ^ ((v & 0x8000u) ? 0xFFFFu : 0x8000u)) ^ flip;
}
__device__ inline uint32_t f16_pattern(uint32_t key, uint32_t flip) {
    const uint32_t asc = (key ^ flip) & 0xFFFFu;
    return (asc & 0x8000u) ? (asc ^ 0x8000u) : (~asc & 0xFFFFu);
}

// Range-checked buffer access: a load past the resource's byte count returns
// 0 and a store past it is dropped by the hardware, so tile edges need no
// per-element predicates and a stray index cannot leave its row.
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer resource word 3 (raw, no swizzle)

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

// Cache-policy bits of the streaming loads and stores (gfx940+: 1 = sc0,
// 2 = nt, 16 = sc1); 0 = default caching.
#ifndef LRS_LOAD_POLICY
#define LRS_LOAD_POLICY 0
#endif
#ifndef LRS_STORE_POLICY
#define LRS_STORE_POLICY 0
#endif

template <typename T> struct BufIO;
template <> struct BufIO<uint32_t> {
    __device__ static inline uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t i) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(i * 4u), 0, LRS_LOAD_POLICY);
    }
    __device__ static inline void store(__amdgpu_buffer_rsrc_t r, uint32_t i, uint32_t v) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, static_cast<int>(i * 4u), 0, LRS_STORE_POLICY);
    }
};
template <> struct BufIO<uint16_t> {
    __device__ static inline uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t i) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(i * 2u), 0, LRS_LOAD_POLICY);
    }
    __device__ static inline void store(__amdgpu_buffer_rsrc_t r, uint32_t i, uint32_t v) {
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(v), r, static_cast<int>(i * 2u), 0,
                                              LRS_STORE_POLICY);
    }
};
template <> struct BufIO<uint64_t> {
    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
    __device__ static inline uint64_t load(__amdgpu_buffer_rsrc_t r, uint32_t i) {
        const v2u w = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(i * 8u), 0, LRS_LOAD_POLICY);
        return (static_cast<uint64_t>(w.y) << 32) | w.x;
    }
    __device__ static inline void store(__amdgpu_buffer_rsrc_t r, uint32_t i, uint64_t v) {
        const v2u w = {static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32)};
        __builtin_amdgcn_raw_buffer_store_b64(w, r, static_cast<int>(i * 8u), 0, LRS_STORE_POLICY);
    }
};
template <> struct BufIO<int64_t> {
    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
    __device__ static inline void store(__amdgpu_buffer_rsrc_t r, uint32_t i, uint32_t v) {
        const v2u w = {v, 0u};
        __builtin_amdgcn_raw_buffer_store_b64(w, r, static_cast<int>(i * 8u), 0, LRS_STORE_POLICY);
    }
};

// Keeps a value materialised in a register at this point (stops the compiler
// from sinking its computation and keeping the operands alive instead).
__device__ inline void pin(uint32_t &v) { asm volatile("" : "+v"(v)); }

// Store v as element i of a row too long for a buffer resource (row is the
// same for the whole workgroup).  With kOff32 (every byte offset of the row
// fits in 32 bits) the address is the row's scalar base plus a 32-bit byte
// offset, which the store adds itself; otherwise a 64-bit address.
template <bool kOff32, typename T>
__device__ inline void wide_store(T *row, uint32_t i, T v) {
    if constexpr (kOff32)
        *reinterpret_cast<T *>(reinterpret_cast<char *>(row) + i * static_cast<uint32_t>(sizeof(T))) = v;
    else
        row[i] = v;
}

// --------------------------------------------------------- wave utilities

// Lanes of this wave whose digit equals this lane's digit (all 64 lanes must
// be active).  For each of the digit's B bits the ballot gives the lanes with
// the bit set; XNOR with this lane's bit spread to all 32 bits (0 or ~0) keeps
// the lanes that agree in that bit, and the match mask is the AND of those
// over all bits.  v_bitop3 does the XNOR and the AND in one instruction: with
// operands (spread, acc, ballot) the table 0x84 is acc & ~(spread ^ ballot).
// The ballots are taken from the spreads themselves (one compare each; the
// pin stops the compiler from deriving them from d with a shift and a compare
// instead), all before the accumulation, so each lands in its own scalar
// register pair and no compare waits on the one before it.
template <int B>
__device__ inline uint64_t match_mask(uint32_t d) {
    uint32_t spread[B];
    uint64_t bal[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
        spread[i] = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(d), i, 1));
        pin(spread[i]);
    }
#pragma unroll
    for (int i = 0; i < B; ++i) bal[i] = __builtin_amdgcn_ballot_w64(spread[i] != 0u);
    uint32_t lo = ~0u, hi = ~0u;
#pragma unroll
    for (int i = 0; i < B; ++i) {
        lo = __builtin_amdgcn_bitop3_b32(spread[i], lo, static_cast<uint32_t>(bal[i]), 0x84);
        hi = __builtin_amdgcn_bitop3_b32(spread[i], hi, static_cast<uint32_t>(bal[i] >> 32), 0x84);
    }
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Number of set bits of m at lanes below this lane.
__device__ inline uint32_t count_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// This lane's rank among the lanes of its digit group (the group members at
// lower lanes), and the group's size, from the group's member mask.
__device__ inline void group_rank(uint64_t members, uint32_t &below, uint32_t &size) {
    below = count_below(members);
    size = static_cast<uint32_t>(__popcll(members));
}

// Stable rank of a wave's ITEMS digits per lane, items in order of j, then of
// lane: out(j, d, r) receives item j's digit d and r = the count of the
// wave's earlier items with digit d, read from the wave's own counters cnt[],
// which advance by each digit group's size (its lowest lane writes).  The
// counter read of item j depends on the write of item j - 1; building the
// match mask of item j + 1 between that read and its use keeps the LDS round
// trip from stalling the wave (the pins inside match_mask hold the read before
// them, and an empty asm that takes the read and the new mask holds its use
// after).  kPipe = false ranks item by item (fewer live registers).
template <int B, int ITEMS, bool kPipe, typename DigitFn, typename OutFn>
__device__ inline void wave_rank(DigitFn digit, uint32_t *cnt, OutFn out) {
    if constexpr (LRS_RANK_PIPELINE && kPipe) {
        uint32_t d = digit(0);
        uint64_t m = match_mask<B>(d);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            uint32_t before = cnt[d];
            uint32_t d_next = 0u;
            uint64_t m_next = 0u;
            if (j + 1 < ITEMS) {
                d_next = digit(j + 1);
                m_next = match_mask<B>(d_next);
                // the read is used only once the next mask is built
                asm volatile("" : "+v"(before) : "v"(static_cast<uint32_t>(m_next)),
                             "v"(static_cast<uint32_t>(m_next >> 32)));
            }
            uint32_t below, size;
            group_rank(m, below, size);
            out(j, d, before + below);
            if (below == 0u) cnt[d] = before + size;
            d = d_next;
            m = m_next;
        }
    } else {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t d = digit(j);
            uint32_t below, size;
            group_rank(match_mask<B>(d), below, size);
            const uint32_t before = cnt[d];
            out(j, d, before + below);
            if (below == 0u) cnt[d] = before + size;
        }
    }
}

// Inclusive sum over the lanes of a wave (all 64 lanes active), by DPP lane
// moves: shifts of 1, 2, 4 and 8 lanes within each row of 16 lanes, then lane
// 15 of each row added to the next row, then lane 31 to the upper half.  No
// LDS round trips (a shuffle-based scan waits on six of them).
template <int kCtrl, int kRowMask>
__device__ inline uint32_t dpp_moved(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, kRowMask, 0xF, false));
}
__device__ inline uint32_t wave_inclusive_scan(uint32_t x) {
    x += dpp_moved<0x111, 0xF>(x);  // row_shr:1
    x += dpp_moved<0x112, 0xF>(x);  // row_shr:2
    x += dpp_moved<0x114, 0xF>(x);  // row_shr:4
    x += dpp_moved<0x118, 0xF>(x);  // row_shr:8
    x += dpp_moved<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_moved<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
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
    const uint32_t *bases;   // this pass's bucket bases of row 0; row r at bases + r * bases_row_stride
    void *status;            // [num_tiles][R] look-back words of this pass
    void *status_next;       // the next pass's words, cleared here (NULL on the last pass)
    uint32_t row_len;        // elements per row
    uint32_t tiles_per_row;
    uint32_t num_tiles;      // rows * tiles_per_row = grid size
    uint32_t bases_row_stride;
    uint32_t shift;          // lowest bit of this pass's digit
    uint32_t digit_mask;     // (1 << width) - 1
    uint64_t flip;           // key transform masks (see KeyTraits)
    uint64_t flip_neg;
    uint32_t spin_limit;     // polls of an unpublished look-back word before the tile counts
                             // its prefix from the keys; 0: always count from the keys
    // Reduce-then-scan (partition) mode: workgroup g sorts tiles
    // [g * part_tiles, (g + 1) * part_tiles) in order, starting digit d at
    // part_offsets[g * R + d] (the output index of its partition's first key
    // of digit d).
    const uint32_t *part_offsets;
    uint32_t part_tiles;
    // Builds with LRS_TILE_TRACE: kTraceWords words per tile of this launch
    // (look-back mode), or NULL; unused otherwise.
    uint64_t *trace;
};

// A tile's trace record: the 100 MHz real-time clock read by thread 0 at the
// start, after the rank, after the local scans, once the offsets are known
// (look-back done, tile reordered), after issuing the key write-out, after the
// payload is in LDS and after issuing the payload write-out (keys-only passes
// repeat the key write-out time), then the XCD id, the HW_ID register
// (CU in bits 8-11, shader engine in 13-15), the workgroup index, and for
// digit 0 the number of predecessors its look-back added up and the polls it
// spent waiting for one to publish.
constexpr int kTraceWords = 12;
enum TraceSlot : int {
    kTrStart = 0, kTrRanked = 1, kTrScanned = 2, kTrOffsets = 3, kTrKeysOut = 4, kTrPayIn = 5, kTrEnd = 6,
    kTrXcc = 7, kTrHwId = 8, kTrBlock = 9, kTrWalk = 10, kTrPolls = 11
};

// Workgroup-wide exclusive scan of one value per thread for a BLOCK-thread
// workgroup.  Every thread must call it.  `tmp` holds BLOCK / 64 words of LDS.
// With kReuse false the caller does not touch `tmp` again before its next
// barrier, so the trailing barrier that protects it is left out.
template <int BLOCK, bool kReuse = true>
__device__ inline uint32_t block_exclusive_scan_n(uint32_t v, uint32_t *tmp, int lane, int wave) {
    constexpr int WAVES = BLOCK / kWave;
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) tmp[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
        if (w < wave) before += tmp[w];
    if (kReuse) __syncthreads();
    return before + inc - v;
}

// The ITEMS consecutive elements from element `first` of a buffer, into one
// thread's registers: with 16-, 8- or 4-byte loads when `vec` (every load in
// range and the buffer's base aligned to the load size), else one load each.
template <typename Stored, int ITEMS, typename Word>
__device__ inline void load_run(Word (&key)[ITEMS], __amdgpu_buffer_rsrc_t r, uint32_t first, bool vec) {
    constexpr uint32_t kBytes = ITEMS * sizeof(Stored);
    static_assert(sizeof(Stored) <= 4 && sizeof(Word) == 4 && kBytes % 4 == 0, "whole words of 4-byte registers");
    constexpr uint32_t kVec = kBytes % 16 == 0 ? 16 : kBytes % 8 == 0 ? 8 : 4;
    if (vec) {
        typedef unsigned int v4u __attribute__((ext_vector_type(4)));
        typedef unsigned int v2u __attribute__((ext_vector_type(2)));
        uint32_t w[kBytes / 4];
        const uint32_t base = first * static_cast<uint32_t>(sizeof(Stored));
#pragma unroll
        for (uint32_t q = 0; q < kBytes / kVec; ++q) {
            const int off = static_cast<int>(base + q * kVec);
            if constexpr (kVec == 16) {
                const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, LRS_LOAD_POLICY);
                w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
            } else if constexpr (kVec == 8) {
                const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, LRS_LOAD_POLICY);
                w[2 * q] = v.x; w[2 * q + 1] = v.y;
            } else {
                w[q] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, LRS_LOAD_POLICY);
            }
        }
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            if constexpr (sizeof(Stored) == 4) key[j] = w[j];
            else key[j] = (w[j / 2] >> (16 * (j % 2))) & 0xFFFFu;
        }
    } else {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) key[j] = BufIO<Stored>::load(r, first + j);
    }
}

// Per-thread counting rank of one tile (digits of at most 4 bits).  Thread t
// holds the tile's elements t * ITEMS .. t * ITEMS + ITEMS - 1 and counts
// their digits (dig(j), padding already mapped to the last digit) in its own
// column of counters cnt[d * BLOCK + t] (R * BLOCK words of LDS); its items of
// one digit rank in item order.  rank[j] = digit << 16 | rank among the
// thread's items of that digit.
#ifndef LRS_COUNT_PAIRS
#define LRS_COUNT_PAIRS 1
#endif
template <uint32_t R, int ITEMS, int BLOCK, typename Dig>
__device__ inline void thread_count_digits(Dig dig, uint32_t (&rank)[ITEMS], uint32_t *cnt, int tid) {
#pragma unroll
    for (uint32_t d = 0; d < R; ++d) cnt[d * BLOCK + tid] = 0u;
    int j = 0;
    if constexpr (LRS_COUNT_PAIRS) {
        // Two items per step: both counters are read before either is
        // written, so each step waits for one LDS round trip instead of two.
        // Items of equal digits: the second ranks one above the first, and
        // the second write (issued after the first) leaves the count at +2.
#pragma unroll
        for (; j + 1 < ITEMS; j += 2) {
            const uint32_t d0 = dig(j), d1 = dig(j + 1);
            const uint32_t c0 = cnt[d0 * BLOCK + tid];
            const uint32_t c1 = cnt[d1 * BLOCK + tid];
            const bool same = d0 == d1;
            cnt[d0 * BLOCK + tid] = c0 + 1u;
            cnt[d1 * BLOCK + tid] = same ? c0 + 2u : c1 + 1u;
            rank[j] = (d0 << 16) | c0;
            rank[j + 1] = (d1 << 16) | (same ? c0 + 1u : c1);
        }
    }
#pragma unroll
    for (; j < ITEMS; ++j) {
        const uint32_t d = dig(j);
        const uint32_t before = cnt[d * BLOCK + tid];
        cnt[d * BLOCK + tid] = before + 1u;
        rank[j] = (d << 16) | before;
    }
}

// The exclusive scan of those counters in (digit, thread) order is the first
// slot of each (digit, thread) group of the tile's digit order, which is
// input order within each digit.  Turns rank[j] into item j's slot, and gives
// thread d < R its digit's count and first slot.  Starts and ends with a
// barrier; after it the counters' LDS is free.
template <uint32_t R, int ITEMS, int BLOCK>
__device__ inline void thread_counts_to_slots(uint32_t (&rank)[ITEMS], uint32_t *cnt, uint32_t *s_tmp, int tid,
                                              int lane, int wave, uint32_t &count, uint32_t &local_start) {
    constexpr uint32_t TILE = static_cast<uint32_t>(BLOCK) * ITEMS;
    __syncthreads();
    // Thread t scans counters [t * R, t * R + R): the thread sums go through
    // a block scan, then the thread's own run.  (16-byte LDS accesses when the
    // run is whole 16-byte words; the run is read twice rather than held,
    // which keeps registers for the keys.)
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    uint32_t sum = 0u;
    if constexpr (R % 4 == 0) {
#pragma unroll
        for (uint32_t i = 0; i < R; i += 4) {
            const v4u v = *reinterpret_cast<const v4u *>(cnt + tid * R + i);
            sum += v.x + v.y + v.z + v.w;
        }
    } else {
#pragma unroll
        for (uint32_t i = 0; i < R; ++i) sum += cnt[tid * R + i];
    }
    uint32_t run = block_exclusive_scan_n<BLOCK, false>(sum, s_tmp, lane, wave);
    if constexpr (R % 4 == 0) {
#pragma unroll
        for (uint32_t i = 0; i < R; i += 4) {
            const v4u v = *reinterpret_cast<const v4u *>(cnt + tid * R + i);
            const uint32_t e0 = run, e1 = e0 + v.x, e2 = e1 + v.y, e3 = e2 + v.z;
            run = e3 + v.w;
            *reinterpret_cast<v4u *>(cnt + tid * R + i) = v4u{e0, e1, e2, e3};
        }
    } else {
#pragma unroll
        for (uint32_t i = 0; i < R; ++i) {
            const uint32_t x = cnt[tid * R + i];
            cnt[tid * R + i] = run;
            run += x;
        }
    }
    __syncthreads();
    if (tid < static_cast<int>(R)) {
        local_start = cnt[tid * BLOCK];
        count = (tid + 1 < static_cast<int>(R) ? cnt[(tid + 1) * BLOCK] : TILE) - local_start;
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t d = rank[j] >> 16;
        rank[j] = cnt[d * BLOCK + tid] + (rank[j] & 0xFFFFu);
    }
    __syncthreads();  // every counter read before the caller reuses the LDS
}

// One LSD pass over one tile of BLOCK * ITEMS elements of one row.
//
// 1. Load the tile's keys (wave-striped: each wave holds a contiguous run of
//    the tile and (item, lane) order is input order).
// 2. Rank stably inside each wave: the lanes sharing a digit are found by
//    ballots; a lane's rank is the wave's running count of its digit plus the group members at
//    lower lanes.
// 3. Per digit: the tile's count (published at once for the look-back; an
//    inclusive count for a row's first tile), the digit's start in the tile,
//    each wave's base inside it, and the row's bucket base.
//    Narrow digits (at most 4 bits) of sweeps with no payload phase replace
//    1-3: each thread loads a run of ITEMS consecutive elements, counts its
//    digits in its own column of LDS counters, and one scan of all counters
//    in (digit, thread) order gives every element's slot and every digit's
//    count and start (no ballots: a few instructions per element).
// 3'. A row-sort pass over 16-bit patterns with the column index as payload
//    (rows of at most 65536) moves one word per element, key << 16 | column:
//    the first pass makes the words at load, the middle passes sort them as
//    plain keys by their high half, the last writes the pattern and column.
// 4. Move every key to its slot of the tile's digit order in LDS, then walk
//    the look-back: the digit's count in earlier tiles of the row, read from
//    the predecessors' published words until an inclusive count is met (or,
//    after a bounded wait, counted from the earlier tiles' keys).
// 5. Publish this tile's inclusive counts, then write the keys (and then the
//    payload through the same slots) with consecutive threads taking
//    consecutive slots, so each digit run goes to consecutive addresses.
//
// With PART set (reduce-then-scan) a workgroup instead sorts the consecutive
// tiles of one partition in order: each tile's digit runs start where the
// previous tile's ended, from offsets a scan of partition counts computed
// before the launch, so nothing is published or waited for.
//
// At least four waves per SIMD (two 512-thread workgroups per CU): the
// partition loop would otherwise take 198 registers and halve that.
template <int B, int ITEMS, int BLOCK, int KK, int PK, typename W, bool PART = false>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(LRS_SWEEP_WAVES_PER_EU))) void sweep_kernel(SweepArgs a) {
    constexpr uint32_t R = 1u << B;
    constexpr int WAVES = BLOCK / kWave;
    constexpr uint32_t TILE = BLOCK * ITEMS;
    static_assert(BLOCK % kWave == 0 && BLOCK >= static_cast<int>(R), "one thread per digit");
    using Stored = typename KeyTraits<KK>::Stored;
    using Word = typename KeyTraits<KK>::Word;
    using St = Status<W>;

    // s_buf holds the tile in digit order (keys, then payload).  Between writing the keys and the payload out of the same slots, each
    // thread keeps its slots' digits in registers, four to a word.
    __shared__ __attribute__((aligned(16))) Word s_buf[TILE];
    uint32_t *const s_pay = reinterpret_cast<uint32_t *>(s_buf);  // the payload's view of the slots
    __shared__ uint32_t s_cnt[WAVES][R];      // per-wave digit counts, then per-wave bases
    __shared__ uint32_t s_goff[R];            // output index of digit run start minus local start
    __shared__ uint32_t s_tmp[WAVES];
    __shared__ uint32_t s_gave_up;            // a look-back wave stopped waiting

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    // 64-bit look-back words also mark rows too long for 32-bit buffer offsets
    constexpr bool kWide = sizeof(W) == 8;
    // Narrow digits of 4-byte words with no separate payload phase rank by
    // per-thread counting over runs of consecutive elements (a few
    // instructions per element) instead of by ballots (4 per digit bit).
    // (Not in partition mode, whose tile loop would need more registers.)
    constexpr bool kBlocked = B <= 4 && !kWide && !PART && sizeof(Word) == 4 &&
                              (PK == kPayNone || PK == kPayPackFirst || PK == kPayUnpackLast);

    // Each wave clears its own row of counters: only that wave touches it
    // until the barrier after the ranking, and one wave's LDS accesses take
    // effect in order, so no workgroup barrier is needed first.  (s_gave_up is
    // read only after two barriers, and set only after the first.)
    for (uint32_t d = lane; d < R; d += kWave) s_cnt[wave][d] = 0u;
    if (!PART && tid == 0) s_gave_up = 0u;

    // Tiles are numbered row-major.  A tile waits below only for earlier tiles
    // of its row, and for a bounded number of polls (see the look-back).
    uint32_t t_first, t_end;
    uint32_t running = 0u;  // partition mode: thread d's output index of the next key of digit d
    if constexpr (PART) {
        t_first = blockIdx.x * a.part_tiles;
        t_end = min(a.num_tiles, t_first + a.part_tiles);
        if (tid < static_cast<int>(R)) running = a.part_offsets[static_cast<uint64_t>(blockIdx.x) * R + tid];
    } else {
        // The tiles of a pass go to the XCDs in chunks of kXcdChunk consecutive
        // tiles (chunk c to XCD c % kXcds); workgroup b runs on XCD b % kXcds,
        // in order of b within its XCD, and takes that XCD's tiles in order.
        // Neighbouring tiles then mostly run on one XCD at the same time, so
        // the cache lines their digit runs share are merged in that XCD's L2
        // instead of being written back partially by two.  The grid is whole
        // rounds of kXcds * kXcdChunk workgroups, so every tile has exactly one
        // (the extra workgroups find none).  A tile waits only for tiles before
        // it, each XCD starts its tiles in order, and waits are bounded.
        const uint32_t x = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
        const uint64_t tile = (static_cast<uint64_t>(k / kXcdChunk) * kXcds + x) * kXcdChunk + k % kXcdChunk;
        t_first = tile < a.num_tiles ? static_cast<uint32_t>(tile) : a.num_tiles;
        t_end = t_first + 1u;
    }
    if (t_first >= a.num_tiles) return;  // a workgroup of the last, partial round
    for (uint32_t t = t_first; t < t_end; ++t) {
        const uint32_t row = t / a.tiles_per_row;
        const uint32_t tile_in_row = t - row * a.tiles_per_row;
        const uint32_t tile_start = tile_in_row * TILE;
        const uint32_t valid = min(TILE, a.row_len - tile_start);
        const uint64_t row_base = static_cast<uint64_t>(row) * a.row_len;

        // (measurement builds only: thread 0 records the tile's phase times)
        auto stamp = [&](int slot) {
            if constexpr (LRS_TILE_TRACE && !PART) {
                if (a.trace != nullptr && tid == 0)
                    a.trace[static_cast<uint64_t>(t) * kTraceWords + slot] = __builtin_amdgcn_s_memrealtime();
            }
        };
        if constexpr (LRS_TILE_TRACE && !PART) {
            if (a.trace != nullptr && tid == 0) {
                uint64_t *rec = a.trace + static_cast<uint64_t>(t) * kTraceWords;
                rec[kTrXcc] = static_cast<uint32_t>(__builtin_amdgcn_s_getreg((3 << 11) | 20));   // XCC_ID
                rec[kTrHwId] = static_cast<uint32_t>(__builtin_amdgcn_s_getreg((31 << 11) | 4));  // HW_ID
                rec[kTrBlock] = blockIdx.x;
            }
        }
        stamp(kTrStart);
        const Stored *kin = static_cast<const Stored *>(a.keys_in) + row_base + tile_start;
        const uint32_t wbase = static_cast<uint32_t>(wave) * kWave * ITEMS;
        const __amdgpu_buffer_rsrc_t kin_rsrc = make_rsrc(kin, valid * sizeof(Stored));

        // 1. Keys.  Elements past the end of the row read as 0 and take the
        // largest digit: last in input order, they rank after every real key of
        // that digit and are never written.  Item j of this thread is tile
        // element elem(j): wave-striped, or the thread's own run of ITEMS
        // consecutive elements for the per-thread counting rank.
        auto elem = [&](int j) -> uint32_t {
            return kBlocked ? static_cast<uint32_t>(tid) * ITEMS + j : wbase + j * kWave + lane;
        };
        Word key[ITEMS];
        if constexpr (kBlocked) {
            const bool vec = valid == TILE && (reinterpret_cast<uintptr_t>(kin) & 15u) == 0u;
            load_run<Stored, ITEMS>(key, kin_rsrc, elem(0), vec);
        } else {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) key[j] = BufIO<Stored>::load(kin_rsrc, elem(j));
        }
        // A first row-sort pass makes the words key << 16 | column at once;
        // from here on its registers hold u32 words whose digits sit 16 bits up.
        if constexpr (PK == kPayPackFirst) {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j)
                key[j] = (f16_key(key[j], static_cast<uint32_t>(a.flip)) << 16) | (tile_start + elem(j));
        }
        // Digit d's first output index in the row (bucket base), thread d.
        uint32_t bucket_base = 0u;
        if (!PART && tid < static_cast<int>(R))
            bucket_base = a.bases[static_cast<uint64_t>(row) * a.bases_row_stride + tid];

        // The pass digit of a key held in registers or LDS.
        auto reg_digit = [&](Word v) -> uint32_t {
            if constexpr (PK == kPayPackFirst)
                return __builtin_amdgcn_ubfe(static_cast<uint32_t>(v), 16u + a.shift,
                                             static_cast<uint32_t>(__builtin_popcount(a.digit_mask)));
            else
                return digit_of<KK>(v, a.flip, a.flip_neg, a.shift, a.digit_mask);
        };

        uint32_t rank[ITEMS];  // digit << 16 | rank within the wave's (or thread's) items of the digit
        uint32_t count = 0u;   // thread d < R: digit d's count in the tile
        uint32_t local_start = 0u;  // thread d < R: digit d's first slot in the tile
        if constexpr (kBlocked) {
            // 2'. Per-thread counting rank (narrow digits), over the tile
            // buffer, which is free until the reorder.
            uint32_t *cnt = reinterpret_cast<uint32_t *>(s_buf);
            static_assert(R * BLOCK * sizeof(uint32_t) <= sizeof(s_buf), "the counters fit the tile buffer");
            if (valid == TILE)
                thread_count_digits<R, ITEMS, BLOCK>([&](int j) { return reg_digit(key[j]); }, rank, cnt, tid);
            else
                thread_count_digits<R, ITEMS, BLOCK>(
                    [&](int j) { return elem(j) >= valid ? R - 1u : reg_digit(key[j]); }, rank, cnt, tid);
            stamp(kTrRanked);
            thread_counts_to_slots<R, ITEMS, BLOCK>(rank, cnt, s_tmp, tid, lane, wave, count, local_start);
            stamp(kTrScanned);
        } else {
            // 2. Stable rank inside the wave; the group's lowest lane advances the
            // wave's running count of the digit.
            // Only a row's last tile has elements past the end, so full tiles take a
            // copy of the loop without the bounds test.
            // (8-byte keys and wide rows rank item by item: the pipelined
            // rank's extra live registers make them spill)
            auto rank_items = [&](auto partial) {
                wave_rank<B, ITEMS, sizeof(Word) == 4 && !kWide>(
                    [&](int j) {
                        const uint32_t dig = reg_digit(key[j]);
                        return (decltype(partial)::value && elem(j) >= valid) ? (R - 1u) : dig;
                    },
                    s_cnt[wave], [&](int j, uint32_t d, uint32_t r) {
                        rank[j] = (d << 16) | r;
                        pin(rank[j]);
                    });
            };
            if (valid == TILE) rank_items(std::false_type{});
            else rank_items(std::true_type{});
            __syncthreads();
            stamp(kTrRanked);

            // 3. Digit d is owned by thread d.
            if (tid < static_cast<int>(R)) {
#pragma unroll
                for (int w = 0; w < WAVES; ++w) {
                    const uint32_t c = s_cnt[w][tid];
                    s_cnt[w][tid] = count;
                    count += c;
                }
            }
        }
        uint32_t real = count;  // padding is not part of the count of the last digit
        if (tid == static_cast<int>(R) - 1) real -= TILE - valid;
        W *status = static_cast<W *>(a.status) + static_cast<uint64_t>(t) * R;
        if (!PART && tid < static_cast<int>(R))
            publish(status + tid, static_cast<W>((tile_in_row == 0 ? St::kInclusive : St::kAggregate) |
                                                 static_cast<W>(real)));
        if constexpr (!kBlocked) {
            // (s_tmp is written again only by the next tile, after three barriers)
            local_start = block_exclusive_scan_n<BLOCK, false>(count, s_tmp, lane, wave);
            if (tid < static_cast<int>(R)) {
#pragma unroll
                for (int w = 0; w < WAVES; ++w) s_cnt[w][tid] += local_start;
            }
            __syncthreads();
            stamp(kTrScanned);

            // 4. Local reorder: every key to its slot.
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const uint32_t d = rank[j] >> 16;
                const uint32_t slot = s_cnt[wave][d] + (rank[j] & 0xFFFFu);
                s_buf[slot] = key[j];
                rank[j] = slot;
            }
        } else {
            // 4. Local reorder: every key to its slot.
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) s_buf[rank[j]] = key[j];
        }
        // Look-back walk, one thread per digit.  Each round trip a lane reads its
        // digit's words of the next kLookback predecessors (nearest first) and adds
        // counts until an inclusive count or an unpublished word.  Lanes of a wave
        // walk together; when none of a wave's lanes finds anything published, one
        // lane polls a single word (with a short sleep) until the predecessor has
        // published, instead of all of them re-reading memory.  The row's first
        // tile publishes an inclusive count at once, so no walk leaves the row.
        //
        // Waiting is bounded: after spin_limit polls the wave gives up, and the
        // workgroup counts the digit over the row's keys before this tile instead
        // (the exact exclusive prefix, at the cost of reading them).  So no tile
        // waits forever, whatever order the hardware starts workgroups in.
        if constexpr (PART) {
            if (tid < static_cast<int>(R)) {
                s_goff[tid] = running - local_start;
                running += real;
            }
        } else {
            W excl = 0;
            const bool from_keys = a.spin_limit == 0u && tile_in_row != 0u;
            bool done = tile_in_row == 0 || from_keys || tid >= static_cast<int>(R);
            bool gave_up = false;  // uniform in the wave
            uint32_t polls = 0;
            uint32_t back = 1;  // the next predecessor to consume is tile t - back
            const W *row_status = static_cast<const W *>(a.status) + tid;
            auto status_of = [&](uint32_t tp) -> W { return observe(row_status + static_cast<uint64_t>(tp) * R); };
            for (;;) {
                const uint64_t walking = __builtin_amdgcn_ballot_w64(!done);
                if (walking == 0 || gave_up) break;
                W sv[kLookback];
#pragma unroll
                for (int i = 0; i < kLookback; ++i)
                    sv[i] = (!done && back + i <= tile_in_row) ? status_of(t - back - i) : W(0);
                uint32_t used = 0;
#pragma unroll
                for (int i = 0; i < kLookback; ++i) {
                    const W flag = sv[i] & ~St::kMask;
                    if (done || used != static_cast<uint32_t>(i) || flag == 0) break;
                    excl += sv[i] & St::kMask;
                    used = i + 1;
                    done = flag == St::kInclusive;
                }
                back += used;
                if (__builtin_amdgcn_ballot_w64(used != 0) == 0) {
                    const int leader = __builtin_ctzll(walking);
                    for (;;) {
                        if (++polls > a.spin_limit) {
                            gave_up = true;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                        W pv = 0;
                        if (lane == leader) pv = status_of(t - back);
                        if (__builtin_amdgcn_ballot_w64(lane == leader && (pv & ~St::kMask) != 0) != 0) break;
                    }
                }
            }
            // The digits a wave found publish their inclusive counts and run
            // starts at once.  If any wave gave up (or no wave looked back), the
            // barrier makes that visible and the workgroup counts every digit
            // over the earlier tiles' keys, which gives the same prefixes, and
            // sets (and publishes) them all again.
            auto finish = [&](W prefix) {
                if (tile_in_row != 0) publish(status + tid, static_cast<W>(St::kInclusive | (prefix + real)));
                s_goff[tid] = bucket_base + static_cast<uint32_t>(prefix) - local_start;
                if (a.status_next != nullptr) static_cast<W *>(a.status_next)[static_cast<uint64_t>(t) * R + tid] = 0;
            };
            if constexpr (LRS_TILE_TRACE) {
                if (a.trace != nullptr && tid == 0) {
                    a.trace[static_cast<uint64_t>(t) * kTraceWords + kTrWalk] = back - 1u;
                    a.trace[static_cast<uint64_t>(t) * kTraceWords + kTrPolls] = polls;
                }
            }
            if (gave_up && lane == 0) s_gave_up = 1u;
            if (!from_keys && !gave_up && tid < static_cast<int>(R)) finish(excl);
            __syncthreads();
            if (from_keys || s_gave_up != 0u) {
                uint32_t *cnt = &s_cnt[0][0];  // free once the tile is reordered
                if (tid < static_cast<int>(R)) cnt[tid] = 0u;
                __syncthreads();
                const Stored *row_keys = static_cast<const Stored *>(a.keys_in) + row_base;
                for (uint32_t i = tid; i < tile_start; i += BLOCK) {
                    const uint32_t d = digit_of<KK>(row_keys[i], a.flip, a.flip_neg, a.shift, a.digit_mask);
                    atomicAdd(&cnt[d], 1u);
                }
                __syncthreads();
                if (tid < static_cast<int>(R)) finish(cnt[tid]);
                __syncthreads();
            }
        }
        if constexpr (PART) __syncthreads();
        stamp(kTrOffsets);

        // 5. Keys out: slot k goes to s_goff[d] + k.  That is below row_len for
        // every real element; the range check of the buffer store only keeps a
        // logic error from becoming a stray store.
        constexpr bool kPayPhase = PK == kPayU32 || PK == kPayIdxFirst || PK == kPayIdxLast;
        constexpr bool kWords = PK == kPayPackFirst || PK == kPayUnpackLast;
        static_assert(!kWords || !kWide, "rows of packed words are short");
        Stored *kout = static_cast<Stored *>(a.keys_out) + row_base;
        uint32_t slot_digits[(ITEMS + 3) / 4];
#pragma unroll
        for (int i = 0; i < (ITEMS + 3) / 4; ++i) slot_digits[i] = 0u;
        // the key outputs: patterns or words as read, packed words (first
        // pass), or the pattern and the int64 column (last pass)
        const __amdgpu_buffer_rsrc_t kout_rsrc =
            PK == kPayPackFirst  ? make_rsrc(static_cast<uint32_t *>(a.keys_out) + row_base, a.row_len * 4u)
            : PK == kPayUnpackLast ? make_rsrc(static_cast<uint16_t *>(a.keys_out) + row_base, a.row_len * 2u)
                                   : make_rsrc(kout, kWide ? 0u : a.row_len * sizeof(Stored));
        const __amdgpu_buffer_rsrc_t iout_rsrc =
            make_rsrc(static_cast<int64_t *>(a.vals_out) + (PK == kPayUnpackLast ? row_base : 0u),
                      PK == kPayUnpackLast ? a.row_len * 8u : 0u);
        // Without the bounds select (full tiles) the loop has no branches and
        // all of a thread's slot reads can be in flight at once.
        auto keys_out = [&](auto partial, auto off32) {
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const uint32_t k = i * BLOCK + tid;
                const Word v = s_buf[k];
                const uint32_t d = reg_digit(v);
                if constexpr (kPayPhase) slot_digits[i / 4] |= d << (8 * (i % 4));
                uint32_t dst;
                if constexpr (decltype(partial)::value) dst = (k < valid) ? s_goff[d] + k : 0xFFFFFFFFu;
                else dst = s_goff[d] + k;
                if constexpr (PK == kPayPackFirst) {
                    BufIO<uint32_t>::store(kout_rsrc, dst, static_cast<uint32_t>(v));
                } else if constexpr (PK == kPayUnpackLast) {
                    BufIO<uint16_t>::store(kout_rsrc, dst, f16_pattern(static_cast<uint32_t>(v) >> 16,
                                                                       static_cast<uint32_t>(a.flip)));
                    BufIO<int64_t>::store(iout_rsrc, dst, static_cast<uint32_t>(v) & 0xFFFFu);
                } else if constexpr (kWide) {
                    // (every slot of a full tile holds a real element)
                    if (!decltype(partial)::value || dst < a.row_len)
                        wide_store<decltype(off32)::value>(kout, dst, static_cast<Stored>(v));
                } else {
                    BufIO<Stored>::store(kout_rsrc, dst, v);
                }
            }
        };
        // 8-byte keys: the payload's loads go out before the key write-out and
        // are in flight during it (3% faster on 2^27 f64 pairs; 2% slower on
        // 2^28 u32 pairs, whose payload is loaded after the keys have gone out)
        constexpr bool kPayEarly = LRS_PAYLOAD_EARLY == 1 || (LRS_PAYLOAD_EARLY == 2 && sizeof(Stored) == 8);
        uint32_t val[ITEMS];
        if constexpr (kPayEarly && (PK == kPayU32 || PK == kPayIdxLast)) {
            const uint32_t *vin = static_cast<const uint32_t *>(a.vals_in) + row_base + tile_start;
            const __amdgpu_buffer_rsrc_t vin_rsrc = make_rsrc(vin, valid * 4u);
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) val[j] = BufIO<uint32_t>::load(vin_rsrc, wbase + j * kWave + lane);
        }
        // Wide rows whose byte offsets all fit in 32 bits store through 32-bit
        // offsets (one copy of each loop per address form, no per-slot test).
        const bool keys_off32 = static_cast<uint64_t>(a.row_len) * sizeof(Stored) <= (uint64_t(1) << 32);
        if constexpr (kWide) {
            if (keys_off32) {
                if (valid == TILE) keys_out(std::false_type{}, std::true_type{});
                else keys_out(std::true_type{}, std::true_type{});
            } else {
                if (valid == TILE) keys_out(std::false_type{}, std::false_type{});
                else keys_out(std::true_type{}, std::false_type{});
            }
        } else {
            if (valid == TILE) keys_out(std::false_type{}, std::false_type{});
            else keys_out(std::true_type{}, std::false_type{});
        }
        stamp(kTrKeysOut);

        // Otherwise the payload is loaded only now, after the keys have gone out
        // (loading it before the look-back, to overlap that wait, measured 0.3%
        // slower on uniform 2^28 pairs and 4% slower with AND-of-3 keys).
        if constexpr (!kPayEarly && (PK == kPayU32 || PK == kPayIdxLast)) {
            const uint32_t *vin = static_cast<const uint32_t *>(a.vals_in) + row_base + tile_start;
            const __amdgpu_buffer_rsrc_t vin_rsrc = make_rsrc(vin, valid * 4u);
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) val[j] = BufIO<uint32_t>::load(vin_rsrc, wbase + j * kWave + lane);
        }

        if constexpr (kPayPhase) {
            __syncthreads();
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                uint32_t v;
                if constexpr (PK == kPayIdxFirst) v = tile_start + wbase + j * kWave + lane;
                else v = val[j];
                s_pay[rank[j]] = v;
            }
            __syncthreads();
            stamp(kTrPayIn);
            using OutT = typename std::conditional<PK == kPayIdxLast, int64_t, uint32_t>::type;
            OutT *vout = static_cast<OutT *>(a.vals_out) + row_base;
            const __amdgpu_buffer_rsrc_t vout_rsrc = make_rsrc(vout, kWide ? 0u : a.row_len * sizeof(OutT));
            if constexpr (kWide) {
                // full tiles without the bounds test (no branch per slot)
                auto pay_out = [&](auto partial, auto off32) {
#pragma unroll
                    for (int i = 0; i < ITEMS; ++i) {
                        const uint32_t k = i * BLOCK + tid;
                        const uint32_t d = (slot_digits[i / 4] >> (8 * (i % 4))) & 0xFFu;
                        if (!decltype(partial)::value || k < valid)
                            wide_store<decltype(off32)::value>(vout, s_goff[d] + k, static_cast<OutT>(s_pay[k]));
                    }
                };
                if (static_cast<uint64_t>(a.row_len) * sizeof(OutT) <= (uint64_t(1) << 32)) {
                    if (valid == TILE) pay_out(std::false_type{}, std::true_type{});
                    else pay_out(std::true_type{}, std::true_type{});
                } else {
                    if (valid == TILE) pay_out(std::false_type{}, std::false_type{});
                    else pay_out(std::true_type{}, std::false_type{});
                }
            } else {
#pragma unroll
                for (int i = 0; i < ITEMS; ++i) {
                    const uint32_t k = i * BLOCK + tid;
                    const uint32_t d = (slot_digits[i / 4] >> (8 * (i % 4))) & 0xFFu;
                    const uint32_t dst = (k < valid) ? s_goff[d] + k : 0xFFFFFFFFu;
                    BufIO<OutT>::store(vout_rsrc, dst, s_pay[k]);
                }
            }
        }
        if constexpr (!kPayPhase) stamp(kTrPayIn);
        stamp(kTrEnd);
        if constexpr (PART) {
            // the next tile reuses the LDS: counters cleared, every read of this tile done
            __syncthreads();
            for (uint32_t i = tid; i < WAVES * R; i += BLOCK) (&s_cnt[0][0])[i] = 0u;
            __syncthreads();
        }
    }
}

// ------------------------------------------------- whole-row resident sort

struct ResidentArgs {
    const void *keys_in;
    void *keys_out;
    const void *vals_in;     // u32 payload (pairs), else unused
    void *vals_out;          // u32 payload (pairs) or int64 column index (rows)
    uint32_t row_len;        // elements per row, at most BLOCK * ITEMS
    uint32_t begin_bit;
    uint32_t end_bit;
    uint64_t flip;           // key transform masks (see KeyTraits)
    uint64_t flip_neg;
};

// Payload of the resident sort.
enum ResPay : int { kResNone = 0, kResU32 = 1, kResIndex = 2 };

// Sorts one row (one workgroup per row) by all of its LSD passes inside LDS:
// the row is read once, every pass ranks it stably (wave ballots, per-wave
// digit counts, local digit starts) and moves keys and payload between two LDS
// buffers, and the result is written once.  The ranking is the one of
// sweep_kernel; with the whole row in one tile the earlier-tile counts are
// zero and the digit starts are the row's bucket bases, so no histogram, scan
// or look-back is needed (one launch in all).
template <int B, int ITEMS, int BLOCK, int KK, int PK>
__global__ __launch_bounds__(BLOCK) void resident_sort_kernel(ResidentArgs a) {
    constexpr uint32_t R = 1u << B;
    constexpr int WAVES = BLOCK / kWave;
    constexpr uint32_t TILE = BLOCK * ITEMS;
    static_assert(BLOCK % kWave == 0 && BLOCK >= static_cast<int>(R), "one thread per digit");
    using Stored = typename KeyTraits<KK>::Stored;

    __shared__ Stored s_key[2][TILE];
    __shared__ uint32_t s_val[PK != kResNone ? 2 : 1][PK != kResNone ? TILE : 1];
    __shared__ uint32_t s_cnt[WAVES][R];
    __shared__ uint32_t s_tmp[WAVES];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t row = blockIdx.x;
    const uint32_t n = a.row_len;
    const uint64_t row_base = static_cast<uint64_t>(row) * n;
    const uint32_t wbase = static_cast<uint32_t>(wave) * kWave * ITEMS;

    uint32_t key[ITEMS];
    uint32_t val[ITEMS];
    {
        const __amdgpu_buffer_rsrc_t kin = make_rsrc(static_cast<const Stored *>(a.keys_in) + row_base, n * sizeof(Stored));
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) key[j] = BufIO<Stored>::load(kin, wbase + j * kWave + lane);
        if constexpr (PK == kResU32) {
            const __amdgpu_buffer_rsrc_t vin = make_rsrc(static_cast<const uint32_t *>(a.vals_in) + row_base, n * 4u);
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) val[j] = BufIO<uint32_t>::load(vin, wbase + j * kWave + lane);
        } else if constexpr (PK == kResIndex) {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) val[j] = wbase + j * kWave + lane;
        }
    }

    int cur = 0;
    for (uint32_t shift = a.begin_bit; shift < a.end_bit; shift += B) {
        const uint32_t width = min(static_cast<uint32_t>(B), a.end_bit - shift);
        const uint32_t mask = (1u << width) - 1u;
        if (shift != a.begin_bit) {
            // this pass reads the previous pass's order, wave-striped
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const uint32_t p = wbase + j * kWave + lane;
                key[j] = s_key[cur][p];
                if constexpr (PK != kResNone) val[j] = s_val[cur][p];
            }
        }
        for (uint32_t i = tid; i < WAVES * R; i += BLOCK) (&s_cnt[0][0])[i] = 0u;
        __syncthreads();

        uint32_t rank[ITEMS];
        wave_rank<B, ITEMS, true>(
            [&](int j) {
                const uint32_t p = wbase + j * kWave + lane;
                return (p < n) ? ((KeyTraits<KK>::key(key[j], a.flip, a.flip_neg) >> shift) & mask) : (R - 1u);
            },
            s_cnt[wave], [&](int j, uint32_t d, uint32_t r) {
                rank[j] = (d << 16) | r;
                pin(rank[j]);
            });
        __syncthreads();

        uint32_t count = 0u;
        if (tid < static_cast<int>(R)) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const uint32_t c = s_cnt[w][tid];
                s_cnt[w][tid] = count;
                count += c;
            }
        }
        const uint32_t start = block_exclusive_scan_n<BLOCK>(count, s_tmp, lane, wave);
        if (tid < static_cast<int>(R)) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) s_cnt[w][tid] += start;
        }
        __syncthreads();

        const int nxt = cur ^ 1;
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t slot = s_cnt[wave][rank[j] >> 16] + (rank[j] & 0xFFFFu);
            s_key[nxt][slot] = static_cast<Stored>(key[j]);
            if constexpr (PK != kResNone) s_val[nxt][slot] = val[j];
        }
        cur = nxt;
        __syncthreads();
    }

    // Write the sorted row; slots past the row end (padding) are dropped by
    // the stores' range checks.
    const __amdgpu_buffer_rsrc_t kout = make_rsrc(static_cast<Stored *>(a.keys_out) + row_base, n * sizeof(Stored));
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const uint32_t k = i * BLOCK + tid;
        BufIO<Stored>::store(kout, k, s_key[cur][k]);
    }
    if constexpr (PK == kResU32) {
        const __amdgpu_buffer_rsrc_t vout = make_rsrc(static_cast<uint32_t *>(a.vals_out) + row_base, n * 4u);
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const uint32_t k = i * BLOCK + tid;
            BufIO<uint32_t>::store(vout, k, s_val[cur][k]);
        }
    } else if constexpr (PK == kResIndex) {
        const __amdgpu_buffer_rsrc_t vout = make_rsrc(static_cast<int64_t *>(a.vals_out) + row_base, n * 8u);
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const uint32_t k = i * BLOCK + tid;
            BufIO<int64_t>::store(vout, k, s_val[cur][k]);
        }
    }
}

// ---------------------------------------- whole-row sort of 16-bit keys

struct RowResidentArgs {
    const uint16_t *keys_in;   // rows x row_len fp16/bf16 patterns
    uint16_t *keys_out;
    const uint32_t *pay_in;    // rows x row_len u32 payload (kResU32), else unused
    void *pay_out;             // int64 column index (kResIndex) or u32 payload (kResU32)
    uint32_t rows;
    uint32_t row_len;          // at most BLOCK * ITEMS
    uint32_t flip;             // 0xFFFF: descending
};

// Sorts whole rows of 16-bit float patterns inside LDS, all passes of the
// 16-bit key, one row at a time per workgroup (workgroups loop over rows).
//
// Each element travels as one word, key << 16 | column: the key is computed
// once per row, the column (< 2^16) is the payload, and one LDS buffer holds
// the row between passes.  Slots past the row end hold key 0xFFFF and their
// own position, so in every pass they take the largest digit, rank after every
// real element and are never written out: no pass needs a bounds test.
//
// Per pass: wave ballots rank each word among the words of its digit in its
// wave (lanes of one wave hold consecutive elements, item by item, so (item,
// lane) order is input order), the per-wave digit counts are scanned into
// digit starts, and the words move to their slots of the pass's order in LDS.
// After the last pass the row is in order: values and column indices go out
// with consecutive threads on consecutive slots.
//
// The next row's keys are loaded into registers before the current row is
// ranked, so HBM reads of one row and writes of the previous one overlap the
// ranking of the current one.
#ifndef LRS_ROW_WAVES_PER_EU
#define LRS_ROW_WAVES_PER_EU 6
#endif
#ifndef LRS_ROW_PREFETCH
#define LRS_ROW_PREFETCH 1
#endif
template <int B, int ITEMS, int BLOCK, int PK>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(LRS_ROW_WAVES_PER_EU))) void row_resident_kernel(RowResidentArgs a) {
    constexpr uint32_t R = 1u << B;
    constexpr int WAVES = BLOCK / kWave;
    constexpr uint32_t TILE = BLOCK * ITEMS;
    static_assert(BLOCK % kWave == 0 && BLOCK >= static_cast<int>(R), "one thread per digit");
    static_assert(TILE <= 65536, "columns must fit in 16 bits");
    __shared__ uint32_t s_w[TILE];
    __shared__ uint32_t s_cnt[2][WAVES][R];  // pass p counts in table p & 1 and clears the other
    __shared__ uint32_t s_tmp[WAVES];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t n = a.row_len;
    const uint32_t wbase = static_cast<uint32_t>(wave) * kWave * ITEMS;
    static_assert((16 / B) % 2 == 0, "an even number of passes leaves table 0 cleared for the next row");

    uint32_t row = blockIdx.x;
    if (row >= a.rows) return;
    uint32_t raw[ITEMS];
    auto load_row = [&](uint32_t r) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.keys_in + static_cast<uint64_t>(r) * n, n * 2u);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) raw[j] = BufIO<uint16_t>::load(rs, wbase + j * kWave + lane);
    };
    if (LRS_ROW_PREFETCH) load_row(row);
    for (uint32_t i = tid; i < WAVES * R; i += BLOCK) (&s_cnt[0][0][0])[i] = 0u;
    __syncthreads();

    for (; row < a.rows; row += gridDim.x) {
        if (!LRS_ROW_PREFETCH) load_row(row);
        uint32_t w[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t p = wbase + j * kWave + lane;
            w[j] = ((p < n) ? (f16_key(raw[j], a.flip) << 16) : 0xFFFF0000u) | p;
        }
        if (LRS_ROW_PREFETCH && row + gridDim.x < a.rows) load_row(row + gridDim.x);

#pragma unroll 1
        for (uint32_t shift = 0; shift < 16u; shift += B) {
            const int t = (shift / B) & 1;
            if (shift != 0) {
#pragma unroll
                for (int j = 0; j < ITEMS; ++j) w[j] = s_w[wbase + j * kWave + lane];
            }

            uint32_t rank[ITEMS];  // rank within the wave's digit
            wave_rank<B, ITEMS, true>([&](int j) { return __builtin_amdgcn_ubfe(w[j], 16u + shift, B); }, s_cnt[t][wave],
                                [&](int j, uint32_t, uint32_t r) {
                                    rank[j] = r;
                                    pin(rank[j]);
                                });
            __syncthreads();

            // Digit d is owned by thread d: per-wave counts become per-wave
            // starts, and the other table is cleared for the next pass.
            uint32_t count = 0u;
            if (tid < static_cast<int>(R)) {
#pragma unroll
                for (int v = 0; v < WAVES; ++v) {
                    const uint32_t c = s_cnt[t][v][tid];
                    s_cnt[t][v][tid] = count;
                    s_cnt[t ^ 1][v][tid] = 0u;
                    count += c;
                }
            }
            const uint32_t start = block_exclusive_scan_n<BLOCK, false>(count, s_tmp, lane, wave);
            if (tid < static_cast<int>(R)) {
#pragma unroll
                for (int v = 0; v < WAVES; ++v) s_cnt[t][v][tid] += start;
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < ITEMS; ++j)
                s_w[s_cnt[t][wave][__builtin_amdgcn_ubfe(w[j], 16u + shift, B)] + rank[j]] = w[j];
            __syncthreads();
        }

        // The row in order: slot k holds the k-th element.
        const uint64_t row_base = static_cast<uint64_t>(row) * n;
        const __amdgpu_buffer_rsrc_t kout = make_rsrc(a.keys_out + row_base, n * 2u);
        if constexpr (PK == kResIndex) {
            const __amdgpu_buffer_rsrc_t iout = make_rsrc(static_cast<int64_t *>(a.pay_out) + row_base, n * 8u);
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const uint32_t k = i * BLOCK + tid;
                const uint32_t v = s_w[k];
                BufIO<uint16_t>::store(kout, k, f16_pattern(v >> 16, a.flip));
                BufIO<int64_t>::store(iout, k, v & 0xFFFFu);
            }
        } else {
            const __amdgpu_buffer_rsrc_t pin_r = make_rsrc(a.pay_in + row_base, n * 4u);
            const __amdgpu_buffer_rsrc_t pout = make_rsrc(static_cast<uint32_t *>(a.pay_out) + row_base, n * 4u);
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                const uint32_t k = i * BLOCK + tid;
                const uint32_t v = s_w[k];
                BufIO<uint16_t>::store(kout, k, f16_pattern(v >> 16, a.flip));
                // the payload of the element from column v & 0xFFFF (slots past
                // the row end read 0 and are not stored)
                BufIO<uint32_t>::store(pout, k, BufIO<uint32_t>::load(pin_r, v & 0xFFFFu));
            }
        }
    }
}

// ------------------------------------------------------- digit histograms

struct HistArgs {
    const void *keys;
    uint32_t *hist;          // [rows][passes][R], zero on entry when atomic != 0
    uint32_t row_len;
    uint32_t chunks_per_row; // workgroups per row
    uint32_t passes;
    uint32_t begin_bit;
    uint32_t end_bit;
    uint64_t flip;           // key transform masks (see KeyTraits)
    uint64_t flip_neg;
    uint32_t atomic;         // 1: several workgroups per row accumulate; 0: one writes it
    uint32_t *bases;         // [rows][passes][R] bucket bases written by the row's last workgroup, or NULL
    uint32_t *done;          // [rows] workgroups finished per row, zero on entry (atomic only)
    uint32_t *status0;       // one workgroup per row: the first pass's look-back words, cleared here (or NULL)
    uint32_t status0_row_words;  // 32-bit words of them per row
};

constexpr int kHistMaxCounters = 2048;  // passes * R for every legal (window, b, key width)
constexpr int kHistCopies = LRS_HIST_COPIES;
#ifndef LRS_HIST_UNROLL
#define LRS_HIST_UNROLL 4
#endif
#ifndef LRS_HIST_BLOCK
#define LRS_HIST_BLOCK 1024
#endif
constexpr int kHistBlock = LRS_HIST_BLOCK;  // threads per histogram workgroup
#ifndef LRS_HIST_INTERLEAVE
#define LRS_HIST_INTERLEAVE 0   // 0: one span of the row per workgroup; 1: 4 KiB strips in turn
#endif

// Counts every pass's digit over one share of one row in LDS, from one read of
// the keys with 16-byte loads, then adds the counts to the row's histogram.
// Digits narrower than 8 bits are counted per byte of the key window (one LDS
// add per byte instead of one per pass: LDS adds bound this kernel) and each
// pass's counts are folded from its byte's counts at the end.
// Lane l counts into copy l % kHistCopies of the counters, and the copies of
// one counter sit in consecutive words: with 32 copies a lane's LDS bank
// depends on its lane alone, whatever the digits, and lanes that share a
// digit do not serialise on one address (except lanes l and l + 32).  The
// counting loop is unrolled: each digit costs one bit-field extract, one
// address add and one LDS add whose offset is an immediate.
template <int B, int KK>
__global__ __launch_bounds__(kHistBlock) void histogram_kernel(HistArgs a) {
    constexpr uint32_t R = 1u << B;
    using Stored = typename KeyTraits<KK>::Stored;
    using Word = typename KeyTraits<KK>::Word;
    constexpr uint32_t kPerVec = 16u / sizeof(Stored);
    constexpr int kMaxPasses = (8 * static_cast<int>(sizeof(Stored)) + B - 1) / B;
    static_assert(kMaxPasses * R <= kHistMaxCounters, "counters must fit");
    // counted digits: the passes' own (8-bit digits) or whole bytes of the window
    constexpr bool kBytes = B < 8;
    constexpr uint32_t kCB = kBytes ? 8u : static_cast<uint32_t>(B);  // counted digit width
    constexpr uint32_t kCR = 1u << kCB;
    constexpr int kMaxCounted = kBytes ? static_cast<int>(sizeof(Stored)) : kMaxPasses;
    // half the copies when the counters would not fit in 128 KB (8-bit digits of 64-bit keys)
    constexpr int kCopies = (kMaxCounted * kCR * kHistCopies * 4 <= 131072) ? kHistCopies : kHistCopies / 2;
    constexpr uint32_t kPassWords = kCR * kCopies;
    constexpr int kUnroll = LRS_HIST_UNROLL;  // 16-byte loads each thread has in flight
    __shared__ uint32_t s_h[kMaxCounted * kCR * kCopies];  // 128 KB for u32 keys
    // byte counts summed over the copies, from which the passes' counts fold
    __shared__ uint32_t s_byte[kBytes ? kMaxCounted * kCR : 1];

    const uint32_t row = blockIdx.x / a.chunks_per_row;
    const uint32_t chunk = blockIdx.x - row * a.chunks_per_row;
    const uint32_t total = a.passes * R;
    if (!a.atomic && a.status0 != nullptr) {
        uint32_t *st = a.status0 + static_cast<uint64_t>(row) * a.status0_row_words;
        for (uint32_t i = threadIdx.x; i < a.status0_row_words; i += kHistBlock) st[i] = 0u;
    }
    const uint32_t counted = kBytes ? (a.end_bit - a.begin_bit + 7u) / 8u : a.passes;
    for (uint32_t i = threadIdx.x; i < counted * kPassWords; i += kHistBlock) s_h[i] = 0u;
    __syncthreads();

    uint32_t *mine = s_h + (threadIdx.x % kCopies);
    auto count_key = [&](Word v) {
        const Word k = KeyTraits<KK>::key(v, a.flip, a.flip_neg);
#pragma unroll
        for (int p = 0; p < kMaxCounted; ++p) {
            if (p < static_cast<int>(counted)) {
                const uint32_t shift = a.begin_bit + static_cast<uint32_t>(p) * kCB;
                const uint32_t width = min(kCB, a.end_bit - shift);
                uint32_t d;
                if constexpr (sizeof(Word) == 8) d = static_cast<uint32_t>(k >> shift) & ((1u << width) - 1u);
                else d = __builtin_amdgcn_ubfe(k, shift, width);
                atomicAdd(mine + p * kPassWords + d * kCopies, 1u);
            }
        }
    };
    auto count_vec = [&](const uint4 &w) {
        if constexpr (sizeof(Stored) == 8) {
            count_key((static_cast<uint64_t>(w.y) << 32) | w.x);
            count_key((static_cast<uint64_t>(w.w) << 32) | w.z);
        } else if constexpr (sizeof(Stored) == 4) {
            count_key(w.x); count_key(w.y); count_key(w.z); count_key(w.w);
        } else {
            count_key(w.x & 0xFFFFu); count_key(w.x >> 16);
            count_key(w.y & 0xFFFFu); count_key(w.y >> 16);
            count_key(w.z & 0xFFFFu); count_key(w.z >> 16);
            count_key(w.w & 0xFFFFu); count_key(w.w >> 16);
        }
    };

    // The row splits into a head up to the first 16-byte boundary, whole
    // 16-byte words, and a tail; rows start on an element boundary.
    const Stored *base = static_cast<const Stored *>(a.keys) + static_cast<uint64_t>(row) * a.row_len;
    const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(base) & 15u) / sizeof(Stored);
    const uint32_t head = min(a.row_len, mis != 0u ? kPerVec - mis : 0u);
    const uint32_t nvec = (a.row_len - head) / kPerVec;
    const uint32_t body_end = head + nvec * kPerVec;
    const uint4 *v4 = reinterpret_cast<const uint4 *>(base + head);

#if LRS_HIST_INTERLEAVE
    const uint32_t step = a.chunks_per_row * kHistBlock;
    uint32_t q = chunk * kHistBlock + threadIdx.x;
    const uint32_t q_end = nvec;
#else
    const uint32_t per = (nvec + a.chunks_per_row - 1) / a.chunks_per_row;
    const uint32_t step = kHistBlock;
    uint32_t q = chunk * per + threadIdx.x;
    const uint32_t q_end = min(nvec, chunk * per + per);
#endif
    for (; q + (kUnroll - 1) * step < q_end; q += kUnroll * step) {
        uint4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) w[u] = v4[q + u * step];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) count_vec(w[u]);
    }
    for (; q < q_end; q += step) count_vec(v4[q]);
    if (chunk == 0 && threadIdx.x < head) count_key(static_cast<Word>(base[threadIdx.x]));
    if (chunk == a.chunks_per_row - 1 && body_end + threadIdx.x < a.row_len)
        count_key(static_cast<Word>(base[body_end + threadIdx.x]));
    __syncthreads();

    // this workgroup's count of counted digit i (copies taken in a rotated
    // order so neighbouring threads read different banks)
    auto copies_sum = [&](uint32_t i) {
        const uint32_t p = i / kCR, d = i - p * kCR;
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < kCopies; ++k)
            c += s_h[p * kPassWords + d * kCopies + ((k + i) % kCopies)];
        return c;
    };
    if constexpr (kBytes) {
        for (uint32_t i = threadIdx.x; i < counted * kCR; i += kHistBlock) s_byte[i] = copies_sum(i);
        __syncthreads();
    }
    // this workgroup's count of digit d of pass p (i = p * R + d): with byte
    // counts, the sum over the byte values whose bits at the pass's offset in
    // its byte are d (the other bits of the byte run over every value)
    auto lds_count = [&](uint32_t i) -> uint32_t {
        if constexpr (!kBytes) {
            return copies_sum(i);
        } else {
            const uint32_t p = i / R, d = i - p * R;
            const uint32_t byte = p / (8u / B), off = (p % (8u / B)) * B;
            const uint32_t shift = a.begin_bit + p * B;
            const uint32_t width = min(static_cast<uint32_t>(B), a.end_bit - shift);
            const uint32_t byte_width = min(8u, a.end_bit - (a.begin_bit + byte * 8u));
            const uint32_t free_bits = byte_width - width;
            const uint32_t low_mask = (1u << off) - 1u;
            uint32_t c = 0;
            for (uint32_t t = 0; t < (1u << free_bits); ++t) {
                const uint32_t v = (t & low_mask) | (d << off) | ((t >> off) << (off + width));
                c += s_byte[byte * kCR + v];
            }
            return c;
        }
    };
    uint32_t *out = a.hist + static_cast<uint64_t>(row) * total;
    for (uint32_t i = threadIdx.x; i < total; i += kHistBlock) {
        const uint32_t c = lds_count(i);
        if (a.atomic) {
            if (c) atomicAdd(out + i, c);
        } else {
            out[i] = c;
        }
    }
    if (a.bases == nullptr) return;

    // The bucket bases: the exclusive scan of each pass's counts.  The last
    // workgroup of the row to finish has every count.  The barrier orders this
    // workgroup's count additions before one thread's acquire-release count of
    // finished workgroups; the last one's acquire orders every workgroup's
    // additions before its reads.
    __shared__ uint32_t s_last;
    if (a.atomic) {
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(a.done + row, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                     a.chunks_per_row - 1 ? 1u : 0u;
        __syncthreads();
        if (s_last == 0u) return;
    }
    // Thread t scans counts K t .. K t + K - 1; one scan runs over all passes
    // at once and each pass then subtracts the prefix at its first digit
    // (exact modulo 2^32).
    constexpr uint32_t K = kHistMaxCounters / kHistBlock;
    static_assert(K * kHistBlock == kHistMaxCounters, "K counts per thread cover every pass");
    auto final_count = [&](uint32_t i) -> uint32_t {
        if (i >= total) return 0u;
        return a.atomic ? __hip_atomic_load(out + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : lds_count(i);
    };
    const uint32_t i0 = K * threadIdx.x;
    uint32_t c[K];
    uint32_t sum = 0u;
#pragma unroll
    for (uint32_t k = 0; k < K; ++k) {
        c[k] = final_count(i0 + k);
        sum += c[k];
    }
    __shared__ uint32_t s_scan[kHistBlock / kWave];
    __shared__ uint32_t s_pass_start[kHistMaxCounters / 2];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t e0 = block_exclusive_scan_n<kHistBlock, false>(sum, s_scan, lane, wave);
    uint32_t run = e0;
#pragma unroll
    for (uint32_t k = 0; k < K; ++k) {
        if (i0 + k < total && (i0 + k) % R == 0) s_pass_start[(i0 + k) / R] = run;
        run += c[k];
    }
    __syncthreads();
    uint32_t *bases = a.bases + static_cast<uint64_t>(row) * total;
    run = e0;
#pragma unroll
    for (uint32_t k = 0; k < K; ++k) {
        if (i0 + k < total) bases[i0 + k] = run - s_pass_start[(i0 + k) / R];
        run += c[k];
    }
}

// --------------------------------------------- reduce-then-scan, per pass

struct PartArgs {
    const void *keys;
    uint32_t *counts;        // [partitions][R]: this pass's digit counts, then (scan) start offsets
    uint32_t n;
    uint32_t part_len;       // elements per partition (whole tiles)
    uint32_t partitions;
    uint32_t shift;
    uint32_t digit_mask;
    uint64_t flip, flip_neg;
};

// Upsweep: the pass digit's count over each partition (one workgroup per
// partition), written without atomics.  Lane copies of the counters as in the
// histogram kernel.
template <int B, int KK>
__global__ __launch_bounds__(kHistBlock) void partition_count_kernel(PartArgs a) {
    constexpr uint32_t R = 1u << B;
    constexpr int kCopies = 32;
    using Stored = typename KeyTraits<KK>::Stored;
    __shared__ uint32_t s_c[R * kCopies];
    for (uint32_t i = threadIdx.x; i < R * kCopies; i += kHistBlock) s_c[i] = 0u;
    __syncthreads();
    const uint32_t g = blockIdx.x;
    const uint64_t lo = static_cast<uint64_t>(g) * a.part_len;
    const uint32_t len = static_cast<uint32_t>(min(static_cast<uint64_t>(a.part_len), a.n - lo));
    const Stored *keys = static_cast<const Stored *>(a.keys) + lo;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(keys, len * sizeof(Stored));
    uint32_t *mine = s_c + (threadIdx.x % kCopies);
    constexpr int kUnroll = 8;
    for (uint32_t i = threadIdx.x; i < len; i += kUnroll * kHistBlock) {
        uint32_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = BufIO<Stored>::load(rsrc, i + u * kHistBlock);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (i + u * kHistBlock < len) {
                const uint32_t d = (KeyTraits<KK>::key(v[u], a.flip, a.flip_neg) >> a.shift) & a.digit_mask;
                atomicAdd(mine + d * kCopies, 1u);
            }
    }
    __syncthreads();
    for (uint32_t d = threadIdx.x; d < R; d += kHistBlock) {
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < kCopies; ++k) c += s_c[d * kCopies + ((k + d) % kCopies)];
        a.counts[static_cast<uint64_t>(g) * R + d] = c;
    }
}

// Scan: for each digit, the total over all partitions gives the bucket base
// (exclusive scan over digits); then each partition's start for the digit is
// the base plus the counts of the earlier partitions.  One workgroup, thread d
// owns digit d; counts are replaced by start offsets in place.
template <int B>
__global__ __launch_bounds__(256) void partition_scan_kernel(PartArgs a) {
    constexpr uint32_t R = 1u << B;
    __shared__ uint32_t s_tmp[256 / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    // Both walks go in batches of kBatch partitions, so each round trip to
    // memory carries kBatch loads (in the second walk a store to one batch
    // would otherwise wait for before every load of the next).
    constexpr uint32_t kBatch = 64;
    uint32_t total = 0u;
    if (tid < static_cast<int>(R)) {
        for (uint32_t g0 = 0; g0 < a.partitions; g0 += kBatch) {
            uint32_t c[kBatch];
#pragma unroll
            for (uint32_t i = 0; i < kBatch; ++i)
                c[i] = (g0 + i < a.partitions) ? a.counts[static_cast<uint64_t>(g0 + i) * R + tid] : 0u;
#pragma unroll
            for (uint32_t i = 0; i < kBatch; ++i) total += c[i];
        }
    }
    uint32_t running = block_exclusive_scan_n<256>(total, s_tmp, lane, wave);
    if (tid < static_cast<int>(R)) {
        for (uint32_t g0 = 0; g0 < a.partitions; g0 += kBatch) {
            uint32_t c[kBatch];
#pragma unroll
            for (uint32_t i = 0; i < kBatch; ++i)
                c[i] = (g0 + i < a.partitions) ? a.counts[static_cast<uint64_t>(g0 + i) * R + tid] : 0u;
#pragma unroll
            for (uint32_t i = 0; i < kBatch; ++i) {
                if (g0 + i < a.partitions) a.counts[static_cast<uint64_t>(g0 + i) * R + tid] = running;
                running += c[i];
            }
        }
    }
}

}  // namespace lrs
