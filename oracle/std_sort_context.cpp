// std_sort_context.cpp -- CPU context figure for the benchmark (not the oracle).
//
// CUDA Handbook ch.16 "Radix Sort" compares its GPU sort with the C++ standard
// library's comparison sort on one CPU core.  This times std::sort of u32 keys
// in place, single-threaded, so the benchmark can print the same kind of
// context line next to the oracle's figure.  Only bench.py's CPU-baseline leg
// calls it.
#include <algorithm>
#include <chrono>
#include <cstdint>

extern "C" double std_sort_u32_seconds(uint32_t *keys, uint64_t n) {
    const auto t0 = std::chrono::steady_clock::now();
    std::sort(keys, keys + n);
    const auto t1 = std::chrono::steady_clock::now();
    return std::chrono::duration<double>(t1 - t0).count();
}
