/*
 * lrs_oracle.c -- plain, slow, single-threaded CPU oracle for LSD radix sort.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the correctness reference that the
 * GPU library is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does. It
 * shares no code, header, table or constant with the HIP library.
 *
 * What it computes (sources are the pages this project is built from):
 *  - One counting-sort pass = histogram the digit, exclusive-scan the counts
 *    into base offsets, then walk the input in order and append each key to its
 *    bucket (CUDA Handbook ch.16 "Radix Sort", the three per-pass steps and the
 *    host pass of Listing 16-8; DSA CUDA from first principles ch.13, sections
 *    13.1 and 13.2).
 *  - LSD radix sort = one stable pass per b-bit digit, least significant digit
 *    first, histogram and offsets recomputed every pass, ping-ponging buffers
 *    (CUDA Handbook ch.16, Listing 16-9; DSA ch.13 section 13.3; gpu.rocks
 *    "The Whole Sort").  Reading: pass p uses the bit window starting at
 *    begin_bit + p*b, and the last pass is narrower when the window width is
 *    not a multiple of b; the pass count is fixed by the window width, never
 *    by the maximum key.
 *  - A second, independent pass routine walks backwards with an inclusive scan
 *    (100 Days of GPU, Day 35, "The digit width looks free" section); it must
 *    agree exactly with the forward walk.
 *  - The order-preserving map from fp16/bf16 bit patterns to unsigned keys
 *    (Day 35 "Pitfalls": a bijection on the way in; FlagTree PR #1084 passes
 *    the descending flag into that conversion).  Reading: negative patterns are
 *    bit-complemented, non-negative patterns get the sign bit set; descending
 *    is the complement of the ascending key, so ties keep input order.
 *  - The same kind of map for 32- and 64-bit signed integers and binary32 /
 *    binary64 floats, and the stable sort of such keys (with an optional
 *    payload) by their image.
 *
 * Every result here is unique (a stable sort of a fixed sequence has exactly one
 * output), so the GPU path is compared against it element for element.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* ---------------------------------------------------------------- digits */

/* b-bit digit of a key: `width` bits starting at bit `shift`. */
uint32_t oracle_digit_bits(uint32_t key, int shift, int width)
{
    uint64_t mask = (width >= 32) ? 0xFFFFFFFFull : ((1ull << width) - 1ull);
    return (uint32_t)(((uint64_t)key >> shift) & mask);
}

/* Decimal-style digit, (value / place) % base (DSA ch.13, section 13.1). */
uint32_t oracle_digit_place(uint64_t value, uint64_t place, uint32_t base)
{
    return (uint32_t)((value / place) % base);
}

/* --------------------------------------------------------- one stable pass */

/*
 * Counting-sort pass over precomputed digits (digit[i] < radix):
 *   step 1  count[d]  = number of i with digit[i] == d
 *   step 2  offset[d] = sum of count[d'] for d' < d      (exclusive scan)
 *   step 3  walk i = 0..n-1 in input order: dest[i] = next[digit[i]]++
 * count/offset are returned as computed by steps 1 and 2 (offset before the
 * walk advances it).  dest is a permutation of 0..n-1.
 */
int oracle_counting_pass(const uint32_t *digit, uint64_t n, uint32_t radix,
                         uint64_t *count, uint64_t *offset, uint64_t *dest)
{
    if (radix == 0 || (n && (!digit || !dest)) || !count || !offset)
        return ORACLE_EINVAL;
    uint64_t *next = (uint64_t *)malloc(sizeof(uint64_t) * radix);
    if (!next) return ORACLE_ENOMEM;

    for (uint32_t d = 0; d < radix; d++) count[d] = 0;
    for (uint64_t i = 0; i < n; i++) {
        if (digit[i] >= radix) { free(next); return ORACLE_EINVAL; }
        count[digit[i]] += 1;
    }
    uint64_t sum = 0;
    for (uint32_t d = 0; d < radix; d++) {
        offset[d] = sum;
        sum += count[d];
    }
    for (uint32_t d = 0; d < radix; d++) next[d] = offset[d];
    for (uint64_t i = 0; i < n; i++) {
        dest[i] = next[digit[i]];
        next[digit[i]] += 1;
    }
    free(next);
    return ORACLE_OK;
}

/*
 * The same pass by the other route: inclusive scan of the counts, then walk
 * the input from the end, pre-decrementing the digit's end position.
 */
int oracle_counting_pass_backward(const uint32_t *digit, uint64_t n, uint32_t radix,
                                  uint64_t *dest)
{
    if (radix == 0 || (n && (!digit || !dest))) return ORACLE_EINVAL;
    uint64_t *end = (uint64_t *)calloc(radix, sizeof(uint64_t));
    if (!end) return ORACLE_ENOMEM;
    for (uint64_t i = 0; i < n; i++) {
        if (digit[i] >= radix) { free(end); return ORACLE_EINVAL; }
        end[digit[i]] += 1;
    }
    for (uint32_t d = 1; d < radix; d++) end[d] += end[d - 1];
    for (uint64_t i = n; i-- > 0;) {
        end[digit[i]] -= 1;
        dest[i] = end[digit[i]];
    }
    free(end);
    return ORACLE_OK;
}

/*
 * Rank of each element inside its digit group, by definition: the number of
 * earlier elements with the same digit (gpu.rocks "The Whole Sort", the
 * destination rule; DSA ch.13 section 13.2, per-element ranks).  O(n^2): only
 * for tiny inputs.
 */
void oracle_rank_within_digit(const uint32_t *digit, uint64_t n, uint64_t *rank)
{
    for (uint64_t i = 0; i < n; i++) {
        uint64_t r = 0;
        for (uint64_t j = 0; j < i; j++)
            if (digit[j] == digit[i]) r++;
        rank[i] = r;
    }
}

/* ------------------------------------------------------------ u32 sorting */

static int check_window(int begin_bit, int end_bit, int key_bits, int digit_bits)
{
    if (digit_bits != 1 && digit_bits != 2 && digit_bits != 4 && digit_bits != 8)
        return 0;
    if (begin_bit < 0 || end_bit > key_bits || begin_bit >= end_bit) return 0;
    return 1;
}

int oracle_num_passes(int begin_bit, int end_bit, int digit_bits)
{
    if (digit_bits <= 0 || end_bit <= begin_bit) return 0;
    return (end_bit - begin_bit + digit_bits - 1) / digit_bits;
}

/*
 * Counts of every pass's digit over the INPUT keys, hist[p * 2^b + d].  The
 * pass-p counts do not depend on the order the keys are in, so these equal the
 * counts each pass of the sort computes.
 */
int oracle_all_pass_histograms(const uint32_t *keys, uint64_t n, int begin_bit,
                               int end_bit, int digit_bits, uint64_t *hist)
{
    if (!check_window(begin_bit, end_bit, 32, digit_bits) || (n && !keys) || !hist)
        return ORACLE_EINVAL;
    int passes = oracle_num_passes(begin_bit, end_bit, digit_bits);
    uint32_t radix = 1u << digit_bits;
    memset(hist, 0, sizeof(uint64_t) * (size_t)passes * radix);
    for (int p = 0; p < passes; p++) {
        int shift = begin_bit + p * digit_bits;
        int width = (end_bit - shift < digit_bits) ? (end_bit - shift) : digit_bits;
        for (uint64_t i = 0; i < n; i++)
            hist[(uint64_t)p * radix + oracle_digit_bits(keys[i], shift, width)] += 1;
    }
    return ORACLE_OK;
}

/*
 * LSD radix sort of u32 keys (and optional u32 payload) by the bit window
 * [begin_bit, end_bit), digit_bits per pass.  Bits outside the window travel
 * with the key but do not order it.  backward != 0 uses the backward-walk pass.
 * Inputs are never written; the result is written to keys_out / vals_out.
 */
int oracle_radix_sort_pairs(const uint32_t *keys_in, const uint32_t *vals_in,
                            uint32_t *keys_out, uint32_t *vals_out, uint64_t n,
                            int begin_bit, int end_bit, int digit_bits, int backward)
{
    if (!check_window(begin_bit, end_bit, 32, digit_bits)) return ORACLE_EINVAL;
    if (n == 0) return ORACLE_OK;
    if (!keys_in || !keys_out || ((vals_in == NULL) != (vals_out == NULL)))
        return ORACLE_EINVAL;

    int passes = oracle_num_passes(begin_bit, end_bit, digit_bits);
    uint32_t radix = 1u << digit_bits;
    int has_vals = vals_in != NULL;

    uint32_t *ka = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *kb = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *va = has_vals ? (uint32_t *)malloc(sizeof(uint32_t) * n) : NULL;
    uint32_t *vb = has_vals ? (uint32_t *)malloc(sizeof(uint32_t) * n) : NULL;
    uint32_t *digit = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint64_t *dest = (uint64_t *)malloc(sizeof(uint64_t) * n);
    uint64_t *count = (uint64_t *)malloc(sizeof(uint64_t) * radix);
    uint64_t *offset = (uint64_t *)malloc(sizeof(uint64_t) * radix);
    int rc = ORACLE_OK;
    if (!ka || !kb || !digit || !dest || !count || !offset || (has_vals && (!va || !vb))) {
        rc = ORACLE_ENOMEM;
        goto done;
    }
    memcpy(ka, keys_in, sizeof(uint32_t) * n);
    if (has_vals) memcpy(va, vals_in, sizeof(uint32_t) * n);

    for (int p = 0; p < passes; p++) {
        int shift = begin_bit + p * digit_bits;
        int width = (end_bit - shift < digit_bits) ? (end_bit - shift) : digit_bits;
        for (uint64_t i = 0; i < n; i++) digit[i] = oracle_digit_bits(ka[i], shift, width);
        rc = backward ? oracle_counting_pass_backward(digit, n, radix, dest)
                      : oracle_counting_pass(digit, n, radix, count, offset, dest);
        if (rc != ORACLE_OK) goto done;
        for (uint64_t i = 0; i < n; i++) kb[dest[i]] = ka[i];
        if (has_vals)
            for (uint64_t i = 0; i < n; i++) vb[dest[i]] = va[i];
        /* ping-pong: the pass output is the next pass input */
        uint32_t *t = ka; ka = kb; kb = t;
        t = va; va = vb; vb = t;
    }
    memcpy(keys_out, ka, sizeof(uint32_t) * n);
    if (has_vals) memcpy(vals_out, va, sizeof(uint32_t) * n);

done:
    free(ka); free(kb); free(va); free(vb);
    free(digit); free(dest); free(count); free(offset);
    return rc;
}

/*
 * Output position of input element i under the stable sort by the windowed
 * key, by definition: the number of elements with a smaller windowed key plus
 * the number of earlier elements with an equal one.  O(n) per element; used to
 * check sampled outputs of sorts too large to run through the full oracle.
 */
uint64_t oracle_stable_position(const uint32_t *keys, uint64_t n, int begin_bit,
                                int end_bit, uint64_t i)
{
    int width = end_bit - begin_bit;
    uint32_t ki = oracle_digit_bits(keys[i], begin_bit, width);
    uint64_t pos = 0;
    for (uint64_t j = 0; j < n; j++) {
        uint32_t kj = oracle_digit_bits(keys[j], begin_bit, width);
        if (kj < ki || (kj == ki && j < i)) pos++;
    }
    return pos;
}

/* ------------------------------------------------------ typed 32-bit keys */

/*
 * Order-preserving u32 image of a 32-bit key (100 Days of GPU, Day 35,
 * "Pitfalls": floats and signed integers sort as unsigned integers after a
 * bijection on the way in).  key_type 0 = u32: the value.  1 = i32: adding 2^31
 * modulo 2^32 carries INT32_MIN..INT32_MAX onto 0..UINT32_MAX in order.
 * 2 = f32 (IEEE binary32, sign-magnitude): a negative pattern is complemented,
 * so larger magnitudes come first, and a non-negative one gets its sign bit
 * set, so it lands above every negative.  Descending: the complement of the
 * ascending image, so equal keys keep their input order.  Readings: -0 sorts
 * just before +0; NaN patterns sort by their image, beyond the infinities.
 */
int oracle_key32(uint32_t bits, int key_type, int descending, uint32_t *out)
{
    uint32_t asc;
    if (key_type == 0) {
        asc = bits;
    } else if (key_type == 1) {
        asc = bits + 0x80000000u;
    } else if (key_type == 2) {
        asc = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
    } else {
        return ORACLE_EINVAL;
    }
    *out = descending ? ~asc : asc;
    return ORACLE_OK;
}

/*
 * Stable sort of n typed 32-bit keys (and an optional u32 payload) by the bit
 * window [begin_bit, end_bit) of their image: the (image, input index) pairs go
 * through the LSD oracle above, then the original key bits and payloads are
 * gathered in the sorted index order.
 */
int oracle_radix_sort_typed(const uint32_t *keys_in, const uint32_t *vals_in, uint32_t *keys_out,
                            uint32_t *vals_out, uint64_t n, int key_type, int descending,
                            int begin_bit, int end_bit, int digit_bits)
{
    if (!check_window(begin_bit, end_bit, 32, digit_bits) || n > 0xFFFFFFFFull) return ORACLE_EINVAL;
    if (n == 0) return ORACLE_OK;
    if (!keys_in || !keys_out || ((vals_in == NULL) != (vals_out == NULL))) return ORACLE_EINVAL;
    uint32_t *image = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *index = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *image_sorted = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *index_sorted = (uint32_t *)malloc(sizeof(uint32_t) * n);
    int rc = ORACLE_OK;
    if (!image || !index || !image_sorted || !index_sorted) { rc = ORACLE_ENOMEM; goto done; }
    for (uint64_t i = 0; i < n; i++) {
        rc = oracle_key32(keys_in[i], key_type, descending, &image[i]);
        if (rc != ORACLE_OK) goto done;
        index[i] = (uint32_t)i;
    }
    rc = oracle_radix_sort_pairs(image, index, image_sorted, index_sorted, n, begin_bit, end_bit,
                                 digit_bits, 0);
    if (rc != ORACLE_OK) goto done;
    for (uint64_t i = 0; i < n; i++) {
        keys_out[i] = keys_in[index_sorted[i]];
        if (vals_in) vals_out[i] = vals_in[index_sorted[i]];
    }
done:
    free(image); free(index); free(image_sorted); free(index_sorted);
    return rc;
}

/*
 * The same maps for 64-bit keys: key_type 3 = u64 (the value), 4 = i64 (add
 * 2^63 modulo 2^64), 5 = f64 (IEEE binary64: complement negative patterns,
 * set the sign bit of the others).  Descending: the complement.
 */
int oracle_key64(uint64_t bits, int key_type, int descending, uint64_t *out)
{
    const uint64_t top = 0x8000000000000000ull;
    uint64_t asc;
    if (key_type == 3) {
        asc = bits;
    } else if (key_type == 4) {
        asc = bits + top;
    } else if (key_type == 5) {
        asc = (bits & top) ? ~bits : (bits | top);
    } else {
        return ORACLE_EINVAL;
    }
    *out = descending ? ~asc : asc;
    return ORACLE_OK;
}

/*
 * Stable LSD sort of n 64-bit keys (optional u32 payload) by the bit window
 * [begin_bit, end_bit) of their image: one counting-sort pass per b-bit digit,
 * low digit first, moving (image, input index); then the original key bits and
 * payloads are gathered in the sorted index order.
 */
int oracle_radix_sort_typed64(const uint64_t *keys_in, const uint32_t *vals_in, uint64_t *keys_out,
                              uint32_t *vals_out, uint64_t n, int key_type, int descending,
                              int begin_bit, int end_bit, int digit_bits)
{
    if (!check_window(begin_bit, end_bit, 64, digit_bits) || n > 0xFFFFFFFFull) return ORACLE_EINVAL;
    if (n == 0) return ORACLE_OK;
    if (!keys_in || !keys_out || ((vals_in == NULL) != (vals_out == NULL))) return ORACLE_EINVAL;
    uint32_t radix = 1u << digit_bits;
    int passes = oracle_num_passes(begin_bit, end_bit, digit_bits);
    uint64_t *img = (uint64_t *)malloc(sizeof(uint64_t) * n);
    uint64_t *img2 = (uint64_t *)malloc(sizeof(uint64_t) * n);
    uint32_t *idx = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *idx2 = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *digit = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint64_t *dest = (uint64_t *)malloc(sizeof(uint64_t) * n);
    uint64_t *count = (uint64_t *)malloc(sizeof(uint64_t) * radix);
    uint64_t *offset = (uint64_t *)malloc(sizeof(uint64_t) * radix);
    int rc = ORACLE_OK;
    if (!img || !img2 || !idx || !idx2 || !digit || !dest || !count || !offset) { rc = ORACLE_ENOMEM; goto done; }
    for (uint64_t i = 0; i < n; i++) {
        rc = oracle_key64(keys_in[i], key_type, descending, &img[i]);
        if (rc != ORACLE_OK) goto done;
        idx[i] = (uint32_t)i;
    }
    for (int p = 0; p < passes; p++) {
        int shift = begin_bit + p * digit_bits;
        int width = (end_bit - shift < digit_bits) ? (end_bit - shift) : digit_bits;
        uint64_t mask = (1ull << width) - 1ull;
        for (uint64_t i = 0; i < n; i++) digit[i] = (uint32_t)((img[i] >> shift) & mask);
        rc = oracle_counting_pass(digit, n, radix, count, offset, dest);
        if (rc != ORACLE_OK) goto done;
        for (uint64_t i = 0; i < n; i++) {
            img2[dest[i]] = img[i];
            idx2[dest[i]] = idx[i];
        }
        uint64_t *ti = img; img = img2; img2 = ti;
        uint32_t *tx = idx; idx = idx2; idx2 = tx;
    }
    for (uint64_t i = 0; i < n; i++) {
        keys_out[i] = keys_in[idx[i]];
        if (vals_in) vals_out[i] = vals_in[idx[i]];
    }
done:
    free(img); free(img2); free(idx); free(idx2); free(digit); free(dest); free(count); free(offset);
    return rc;
}

/* ------------------------------------------------- fp16 / bf16 row sorting */

/*
 * Order-preserving key of a 16-bit float pattern (fp16 1-5-10 and bf16 1-8-7
 * are both sign-magnitude with the exponent above the mantissa, so one map
 * serves both).  Ascending: a negative pattern is complemented (larger
 * magnitude -> smaller key), a non-negative one gets its sign bit set.
 * Descending: the complement of the ascending key.
 */
uint16_t oracle_float16_key(uint16_t bits, int descending)
{
    uint16_t asc = (bits & 0x8000u) ? (uint16_t)(~bits) : (uint16_t)(bits | 0x8000u);
    return descending ? (uint16_t)(~asc) : asc;
}

/*
 * Independent LSD sort of every row of a rows x n matrix of 16-bit float
 * patterns.  The payload is the column index (0..n-1), created here, never an
 * input.  vals_out gets the original bit patterns in sorted order, idx_out the
 * int64 column each came from.
 */
int oracle_segmented_row_sort(const uint16_t *vals_in, uint16_t *vals_out, int64_t *idx_out,
                              int64_t rows, int64_t n, int descending, int digit_bits)
{
    if (!check_window(0, 16, 16, digit_bits) || rows < 0 || n < 0) return ORACLE_EINVAL;
    if (rows == 0 || n == 0) return ORACLE_OK;
    if (!vals_in || !vals_out || !idx_out) return ORACLE_EINVAL;

    uint32_t *key = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *idx = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *key_out = (uint32_t *)malloc(sizeof(uint32_t) * n);
    uint32_t *idx_sorted = (uint32_t *)malloc(sizeof(uint32_t) * n);
    int rc = ORACLE_OK;
    if (!key || !idx || !key_out || !idx_sorted) { rc = ORACLE_ENOMEM; goto done; }

    for (int64_t r = 0; r < rows; r++) {
        const uint16_t *row = vals_in + r * n;
        for (int64_t j = 0; j < n; j++) {
            key[j] = oracle_float16_key(row[j], descending);
            idx[j] = (uint32_t)j;
        }
        rc = oracle_radix_sort_pairs(key, idx, key_out, idx_sorted, (uint64_t)n, 0, 16,
                                     digit_bits, 0);
        if (rc != ORACLE_OK) goto done;
        for (int64_t j = 0; j < n; j++) {
            vals_out[r * n + j] = row[idx_sorted[j]];
            idx_out[r * n + j] = (int64_t)idx_sorted[j];
        }
    }
done:
    free(key); free(idx); free(key_out); free(idx_sorted);
    return rc;
}

/* Per-row, per-pass digit counts of the transformed keys: hist[(r*P + p)*2^b + d]. */
int oracle_segmented_histograms(const uint16_t *vals, int64_t rows, int64_t n,
                                int descending, int digit_bits, uint64_t *hist)
{
    if (!check_window(0, 16, 16, digit_bits) || rows < 0 || n < 0 || !hist) return ORACLE_EINVAL;
    int passes = oracle_num_passes(0, 16, digit_bits);
    uint32_t radix = 1u << digit_bits;
    memset(hist, 0, sizeof(uint64_t) * (size_t)rows * passes * radix);
    for (int64_t r = 0; r < rows; r++)
        for (int p = 0; p < passes; p++)
            for (int64_t j = 0; j < n; j++) {
                uint32_t k = oracle_float16_key(vals[r * n + j], descending);
                hist[((uint64_t)r * passes + p) * radix + oracle_digit_bits(k, p * digit_bits, digit_bits)] += 1;
            }
    return ORACLE_OK;
}

/* Sorted position of element j within its row, by definition (see above). */
uint64_t oracle_row_stable_position(const uint16_t *row, uint64_t n, int descending, uint64_t j)
{
    uint16_t kj = oracle_float16_key(row[j], descending);
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n; i++) {
        uint16_t ki = oracle_float16_key(row[i], descending);
        if (ki < kj || (ki == kj && i < j)) pos++;
    }
    return pos;
}
