/*
 * lsd_radix_sort.h -- C ABI of the MI355X (gfx950) LSD radix sort library.
 *
 * The method: least-significant-digit radix sort.  Each pass histograms one
 * b-bit digit, exclusive-scans the 2^b bucket counts into base offsets and
 * stably scatters the keys (and payload); passes go from the low digit to the
 * high digit, ping-ponging between two buffers (CUDA Handbook ch.16 "Radix
 * Sort", the three per-pass steps; DSA CUDA from first principles ch.13,
 * section 13.3; gpu.rocks "The Whole Sort").
 *
 * Conventions shared by every entry point:
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    allocates, frees and synchronises nothing: every call validates its
 *    arguments on the host, enqueues its kernels on `stream` (a hipStream_t;
 *    NULL = the null stream) and returns.
 *  - Inputs are never written (sorting is out of place; 100 Days of GPU,
 *    Day 35, "Pitfalls").  Outputs must not overlap inputs, each other or the
 *    workspace (LRS_ERR_ALIASING).
 *  - Data pointers are naturally aligned for their element type; the
 *    workspace is 256-byte aligned (torch allocations are); otherwise
 *    LRS_ERR_ALIGNMENT.
 *  - The caller provides scratch device memory (`workspace`) of at least the
 *    size the matching *_workspace_size() call returns; its contents on entry
 *    do not matter and on return are unspecified.  Calls that share a
 *    workspace must be ordered on one stream.  Inputs whose rows hold at most
 *    8192 elements are sorted whole inside one workgroup and need no
 *    workspace (the size is 0 and workspace may be NULL).
 *  - The result of a sort is unique: a stable sort by the key, ties in input
 *    order, payload travelling with its key.
 *  - Return value: LRS_OK or an lrs_status code.  Argument errors are reported
 *    before anything is enqueued.  LRS_ERR_HIP means a kernel launch was
 *    rejected by the runtime; faults during execution surface at the caller's
 *    next synchronisation.  No C++ exception crosses this boundary.
 */
#ifndef LSD_RADIX_SORT_H
#define LSD_RADIX_SORT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lrs_status {
    LRS_OK = 0,
    LRS_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    LRS_ERR_BIT_RANGE = 2,           /* begin_bit/end_bit outside 0 <= begin < end <= key width */
    LRS_ERR_DIGIT_BITS = 3,          /* digit_bits not 1, 2, 4 or 8 */
    LRS_ERR_SIZE = 4,                /* element count or shape beyond the supported limit */
    LRS_ERR_ALIASING = 5,            /* an output overlaps an input, another output or the workspace */
    LRS_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace_bytes below the *_workspace_size() figure */
    LRS_ERR_DTYPE = 7,               /* dtype or key_type not one of the values below */
    LRS_ERR_HIP = 8,                 /* the HIP runtime rejected a launch or query */
    LRS_ERR_ALIGNMENT = 9,           /* a pointer is not aligned as required (see below) */
    LRS_ERR_OPTION = 10              /* a field of the lrs_options argument has an invalid value */
} lrs_status;

#define LRS_DTYPE_FP16 0
#define LRS_DTYPE_BF16 1

/* Key types of radix_sort_keys_typed / radix_sort_pairs_typed. */
#define LRS_KEY_U32 0
#define LRS_KEY_I32 1
#define LRS_KEY_F32 2
#define LRS_KEY_U64 3
#define LRS_KEY_I64 4
#define LRS_KEY_F64 5

/* Largest u32 sort: n < 2^32 elements.  Largest segmented row: n < 2^30
 * (FlagTree PR #1084 caps one row at 2^30 elements). */
#define LRS_MAX_KEYS 0xFFFFFFFFull
#define LRS_MAX_ROW_LEN ((1ull << 30) - 1ull)

/*
 * Per-call options.  Every sort entry point (and the workspace-size queries)
 * takes a `const lrs_options *opts` as its last argument; NULL, or a struct
 * whose fields are all zero, means the defaults.  Options affect only the call
 * they are passed to: the library keeps no global settings.
 *
 * scan_strategy     How single-row sorts (radix_sort_keys/pairs and the typed
 *                   forms) find each tile's output offsets (CUDA Handbook
 *                   ch.16: the scan of the per-block counts; FlagTree PR #1084
 *                   step 2 compares a status look-back with precomputed offsets):
 *       LRS_SCAN_LOOKBACK (0, default)  one launch per pass; each tile publishes
 *           its digit counts and adds up its predecessors' (decoupled look-back).
 *       LRS_SCAN_REDUCE_THEN_SCAN  three launches per pass: count the digit over
 *           each of up to 512 partitions of whole tiles, scan those counts into
 *           start offsets, then sort each partition's tiles in order from them;
 *           the keys are read once more per pass.  Segmented row sorts and
 *           64-bit keys always use the look-back.
 *     The result is identical.  Any other value: LRS_ERR_OPTION.
 * spin_limit        Bound on how long a sweep tile waits for the counts an
 *                   earlier tile of its row publishes, in polls of about a
 *                   microsecond.  A tile that runs out of polls counts its digit
 *                   over the earlier tiles' keys instead (the same result), so
 *                   no launch waits forever whatever order the hardware starts
 *                   workgroups in.  0 = the default, LRS_DEFAULT_SPIN_LIMIT.
 * prefix_from_keys  Nonzero: no tile waits at all; every tile counts its prefix
 *                   from the keys (slow; it exists to test that path).
 * wide_from         0 (default): rows take the sweep with 64-bit look-back words
 *                   and 64-bit store addresses only where they need it (from
 *                   2^30 four-byte keys, from 2^29 eight-byte keys or row-sort
 *                   elements).  Nonzero: rows of at least wide_from elements
 *                   that are sorted by sweeps (more than 8192 elements) take
 *                   it as well (a test hook; the result is identical).  Pass
 *                   the same options to the workspace-size query.
 * timer             If not NULL, every kernel the call enqueues is timed by
 *                   HIP events on its stream and recorded in this timer (see
 *                   radix_sort_timer_create).  A timer must not be used by two
 *                   calls at the same time.  Timing is for calls run eagerly:
 *                   a timed call on a stream that is being captured into a
 *                   graph returns LRS_ERR_OPTION and enqueues nothing.
 */
#define LRS_SCAN_LOOKBACK 0
#define LRS_SCAN_REDUCE_THEN_SCAN 1
#define LRS_DEFAULT_SPIN_LIMIT 65536u

typedef struct lrs_timer lrs_timer;

typedef struct lrs_options {
    int scan_strategy;
    uint32_t spin_limit;
    int prefix_from_keys;
    uint64_t wide_from;
    lrs_timer *timer;
} lrs_options;

/*
 * Bytes of workspace radix_sort_keys (with_values = 0) or radix_sort_pairs
 * (with_values = 1) needs for these arguments.  Returns 0 for arguments the
 * sort would reject, and for n == 0.
 */
size_t radix_sort_workspace_size(uint64_t n, int begin_bit, int end_bit, int digit_bits,
                                 int with_values, const lrs_options *opts);

/*
 * Stable LSD sort of n u32 keys by the bit window [begin_bit, end_bit),
 * digit_bits (b) bits per pass, ceil((end_bit - begin_bit) / b) passes, low
 * digit first; the last pass is narrower when b does not divide the window
 * (CUDA Handbook ch.16, the pass and driver; b in {1, 2, 4, 8} as that page
 * allows).  Bits outside the window travel with the key but do not order it:
 * keys equal inside the window keep their input order.
 *   keys_in   [n] u32, read only          keys_out [n] u32, written
 *   0 <= begin_bit < end_bit <= 32; n < 2^32; n == 0 is a no-op.
 */
int radix_sort_keys(const uint32_t *keys_in, uint32_t *keys_out, uint64_t n, int begin_bit,
                    int end_bit, int digit_bits, void *workspace, size_t workspace_bytes,
                    void *stream, const lrs_options *opts);

/*
 * As radix_sort_keys, carrying one u32 payload per key: vals_out[i] is the
 * payload of the key that lands at keys_out[i] (100 Days of GPU, Day 35,
 * "Exercise": the payload rides along with every move of its key).
 *   vals_in [n] u32, read only            vals_out [n] u32, written
 */
int radix_sort_pairs(const uint32_t *keys_in, const uint32_t *vals_in, uint32_t *keys_out,
                     uint32_t *vals_out, uint64_t n, int begin_bit, int end_bit, int digit_bits,
                     void *workspace, size_t workspace_bytes, void *stream, const lrs_options *opts);

/*
 * As segmented_row_sort, but each element carries a caller-supplied u32
 * payload instead of the column index: pay_out[r][j] is the payload of the
 * element that lands at vals_out[r][j] (the payload rides along with every
 * move of its key).  pay_in / pay_out are row-major rows x n u32, 4-byte
 * aligned, and must not overlap each other, the values or the workspace.  The
 * workspace is segmented_row_sort_workspace_size(rows, n, digit_bits).
 */
int segmented_row_sort_pairs(const uint16_t *vals_in, const uint32_t *pay_in, uint16_t *vals_out,
                             uint32_t *pay_out, int64_t rows, int64_t n, int dtype, int descending,
                             int digit_bits, void *workspace, size_t workspace_bytes, void *stream, const lrs_options *opts);

/*
 * Stable LSD sort of n 32- or 64-bit keys of type key_type, ascending or
 * descending, with or without a u32 payload.  The sort orders the key's
 * order-preserving unsigned image (100 Days of GPU, Day 35, "Pitfalls": a
 * bijection on the way in, so floats and signed integers sort as unsigned
 * integers):
 *   LRS_KEY_U32 / U64  the value itself;
 *   LRS_KEY_I32 / I64  two's complement with the sign bit flipped;
 *   LRS_KEY_F32 / F64  IEEE-754 binary32 / binary64 bits: negative patterns
 *                complemented, non-negative ones with the sign bit set.  So
 *                -0 sorts immediately before +0, and NaNs sort by bit pattern
 *                beyond the infinities (sign-bit-set NaNs first, the others last);
 * descending (nonzero) sorts the complement of that image, so equal keys keep
 * their input order in both directions.  [begin_bit, end_bit) selects bits of
 * the image (0, 32 or 0, 64 for a full sort; end_bit <= the key width).  The
 * stored key bits are what is moved; the outputs hold input values, never
 * transformed ones.  Keys are 4-byte (32-bit types) or 8-byte (64-bit types)
 * elements, aligned to their size; the workspace size comes from
 * radix_sort_typed_workspace_size (for 32-bit types it equals
 * radix_sort_workspace_size).  Pointers, sizes, alignment and errors are
 * otherwise as for radix_sort_keys / radix_sort_pairs; an unknown key_type
 * returns LRS_ERR_DTYPE.  LRS_KEY_U32 ascending is exactly radix_sort_keys /
 * radix_sort_pairs.  64-bit keys always take the multi-launch path (no
 * whole-row resident sort) and the look-back scan strategy.
 */
size_t radix_sort_typed_workspace_size(uint64_t n, int key_type, int begin_bit, int end_bit, int digit_bits,
                                       int with_values, const lrs_options *opts);
int radix_sort_keys_typed(const void *keys_in, void *keys_out, uint64_t n, int key_type, int descending,
                          int begin_bit, int end_bit, int digit_bits, void *workspace,
                          size_t workspace_bytes, void *stream, const lrs_options *opts);
int radix_sort_pairs_typed(const void *keys_in, const uint32_t *vals_in, void *keys_out, uint32_t *vals_out,
                           uint64_t n, int key_type, int descending, int begin_bit, int end_bit,
                           int digit_bits, void *workspace, size_t workspace_bytes, void *stream, const lrs_options *opts);

/* Bytes of workspace segmented_row_sort needs; 0 for rejected arguments or empty input. */
size_t segmented_row_sort_workspace_size(int64_t rows, int64_t n, int digit_bits, const lrs_options *opts);

/*
 * Sort each row of a row-major rows x n matrix of fp16 or bf16 values
 * independently, ascending or descending, returning the sorted values and the
 * int64 column each came from (FlagTree PR #1084: the radix sort behind
 * torch-style sort over the last dimension, with an arange column index as
 * payload).  Keys are the 16-bit patterns through an order-preserving map
 * (100 Days of GPU, Day 35, "Pitfalls"): negative patterns are complemented,
 * non-negative ones get the sign bit set; descending uses the complement of
 * that key, so equal values keep their input order in both directions.
 * -0 sorts immediately before +0 ascending (after it descending); NaNs sort by
 * pattern beyond the infinities.  Passes: 16 / digit_bits.
 *   vals_in  [rows][n] u16 patterns, read only
 *   vals_out [rows][n] u16 patterns, written (the input patterns, permuted)
 *   idx_out  [rows][n] int64 column indices, written
 *   dtype: LRS_DTYPE_FP16 or LRS_DTYPE_BF16; descending: 0 or 1
 *   rows >= 0, 0 <= n <= LRS_MAX_ROW_LEN; rows * n < 2^40.
 */
int segmented_row_sort(const uint16_t *vals_in, uint16_t *vals_out, int64_t *idx_out,
                       int64_t rows, int64_t n, int dtype, int descending, int digit_bits,
                       void *workspace, size_t workspace_bytes, void *stream, const lrs_options *opts);

/*
 * The per-pass digit counts of radix_sort_keys' first kernel: all passes'
 * histograms from one read of the keys (FlagTree PR #1084, step 2 "Before":
 * one kernel counts every pass).  hist_out[p * 2^b + d] = number of keys
 * whose pass-p digit is d.  hist_out is a device array of
 * ceil((end_bit - begin_bit) / b) * 2^b u32, 16-byte aligned, written (not
 * accumulated).
 */
int radix_sort_digit_histograms(const uint32_t *keys, uint64_t n, int begin_bit, int end_bit,
                                int digit_bits, uint32_t *hist_out, void *stream, const lrs_options *opts);

/* Copy `bytes` bytes from src to dst with a plain streaming kernel (the
 * bandwidth yardstick of 100 Days of GPU, Day 35, "Results", the copy row).
 * Both pointers 16-byte aligned, non-overlapping.  Only opts->timer is used. */
int radix_sort_copy_probe(const void *src, void *dst, size_t bytes, void *stream, const lrs_options *opts);

/*
 * radix_sort_pairs for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace argument: its workspace is a device array of
 * LRS_NO_ALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  It calls no hipMalloc, hipFree or other allocating routine.
 * Sizes whose workspace (radix_sort_workspace_size(n, ..., 1, opts)) exceeds
 * the array return LRS_ERR_SIZE: with 8-bit digits over 32 bits, about 8.2
 * million pairs (rows of at most 8192 pairs need no workspace at all).  Every
 * call on one GPU shares that GPU's array, so calls that may run at the same
 * time on one GPU (two streams, two threads) race and corrupt each other's
 * results: order them, or use radix_sort_pairs with workspaces of their own.
 * The first call on each device looks up the array's device address
 * (LRS_ERR_HIP if the runtime cannot give it).  Arguments, result and other
 * errors are those of radix_sort_pairs.
 */
#define LRS_NO_ALLOC_SCRATCH_BYTES (64ull << 20)
int radix_sort_pairs_no_alloc(const uint32_t *keys_in, const uint32_t *vals_in, uint32_t *keys_out,
                              uint32_t *vals_out, uint64_t n, int begin_bit, int end_bit, int digit_bits,
                              void *stream, const lrs_options *opts);

/*
 * Kernel timing for measurement (opts->timer).  radix_sort_timer_create
 * returns a new timer (NULL if host memory runs out); calls given it in their
 * options time each kernel they enqueue with a pair of HIP events on their
 * stream, stamped by the kernel's dispatch itself (a call over at most 65,536
 * elements, or 65,536 four-byte words for the copy probe, records the pair
 * just before and after each launch instead; a reduce-then-scan pass's count
 * and scan kernels share one pair).  The events carry no system-scope fence: they time the work but
 * do not make its results visible to the host (synchronize the stream for
 * that).  radix_sort_timer_read waits for the events and reports, per kernel
 * kind (0 = workspace clear, 1 = digit histogram and the reduce-then-scan
 * count and scan, 2 = sweep/scatter pass, 3 = copy probe, 4 = whole-row
 * resident sort), the summed milliseconds and the number of launches in the
 * two 5-entry arrays (either may be NULL), then empties the timer.  At most
 * 65536 launches are recorded between reads.  radix_sort_timer_destroy frees
 * the timer and its events (NULL is a no-op); no call may still be recording
 * into it.
 */
lrs_timer *radix_sort_timer_create(void);
int radix_sort_timer_read(lrs_timer *timer, double *ms_by_kind, int *launches_by_kind);
void radix_sort_timer_destroy(lrs_timer *timer);

/*
 * Tile phase records for measurement, in libraries built with LRS_TILE_TRACE=1
 * (python -m lsd_radix_sort_amd.build -DLRS_TILE_TRACE=1 --out PATH); the
 * default build returns LRS_ERR_OPTION from radix_sort_timer_trace_tiles and
 * records nothing.  The phases are those of one tile of a sweep pass with a
 * decoupled look-back (CUDA Handbook ch.16: the per-block counting, scan and
 * scatter of a pass; FlagTree PR #1084 step 2: the status look-back).
 *
 * radix_sort_timer_trace_tiles(timer, buf, words) gives the timer a device
 * buffer of `words` 64-bit words (8-byte aligned, owned by the caller, which
 * keeps it alive while calls record into it; buf NULL and words 0 detach it)
 * and restarts its count.  Every later look-back sweep launch of an eager call
 * timed by this timer takes the next num_tiles * LRS_TILE_TRACE_WORDS words
 * while the buffer has room (launches that find no room record nothing), and
 * each tile's first thread writes its record there: words 0-6 the GPU's
 * 100 MHz real-time clock at the tile's start, after the rank, after the local
 * scans, once its output offsets are known (look-back done, tile reordered),
 * after issuing the key write-out, once the payload is in LDS and after issuing
 * the payload write-out (keys-only passes repeat the key write-out time in
 * words 5 and 6); word 7 the XCD id, word 8 the HW_ID register (CU in bits
 * 8-11, shader engine in bits 13-15), word 9 the workgroup index, word 10 the
 * number of predecessor tiles whose counts digit 0's look-back added up, word
 * 11 the polls it spent waiting for a predecessor to publish.  Tile t of a
 * launch is record t, tiles numbered row-major.
 * radix_sort_timer_trace_used stores the words taken since the buffer was set.
 */
#define LRS_TILE_TRACE_WORDS 12
int radix_sort_timer_trace_tiles(lrs_timer *timer, uint64_t *buf, uint64_t words);
int radix_sort_timer_trace_used(const lrs_timer *timer, uint64_t *words);

/* Static description of a status code; never NULL. */
const char *radix_sort_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LSD_RADIX_SORT_H */
