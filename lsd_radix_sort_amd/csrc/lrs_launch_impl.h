// lrs_launch_impl.h -- definitions of the launcher templates declared in
// lrs_launch.h; included only by the lrs_inst_*.hip files, which instantiate
// them (and so compile the kernels) for one key kind each.
#pragma once

#include <atomic>

#include "lrs_launch.h"

namespace lrs {

template <int B, int ITEMS, int BLOCK, int KK, int PK, typename W, bool PART>
void launch_sweep_cfg(const SweepArgs &a, uint64_t grid_size, const Launch &L) {
    // look-back sweeps map tiles from the workgroup index in whole rounds of
    // kXcds * kXcdChunk workgroups (see sweep_kernel); the extra ones return
    constexpr uint64_t round = uint64_t(kXcds) * kXcdChunk;
    if (!PART) grid_size = (grid_size + round - 1) / round * round;
    const dim3 grid(static_cast<uint32_t>(grid_size));
    launch_on(sweep_kernel<B, ITEMS, BLOCK, KK, PK, W, PART>, grid, dim3(BLOCK), L, a);
}

template <int B, int KK, int PK, bool PART>
hipError_t launch_sweep_b(const SweepArgs &a, int cfg, bool wide, uint64_t grid, const Launch &L) {
    constexpr bool k64 = sizeof(typename KeyTraits<KK>::Stored) == 8;
    constexpr bool ko = no_payload_phase(PK);
    constexpr TileCfg c0 = tile_cfg_of(k64, 0, ko), c1 = tile_cfg_of(k64, 1, ko), c2 = tile_cfg_of(k64, 2, ko);
    // 64-bit look-back words (and 64-bit store addressing) only occur for rows
    // of 2^29 or more elements (2^30 for 4-byte keys), which always take the
    // largest tile; rows carried as packed words are at most 65536 long.
    constexpr bool kPacked = PK == kPayPackFirst || PK == kPayUnpackLast;
    if (wide) {
        if constexpr (kPacked) return hipErrorInvalidValue;
        else launch_sweep_cfg<B, c2.items, c2.block, KK, PK, uint64_t, PART>(a, grid, L);
    } else if (cfg == 2)
        launch_sweep_cfg<B, c2.items, c2.block, KK, PK, uint32_t, PART>(a, grid, L);
    else if (cfg == 1)
        launch_sweep_cfg<B, c1.items, c1.block, KK, PK, uint32_t, PART>(a, grid, L);
    else
        launch_sweep_cfg<B, c0.items, c0.block, KK, PK, uint32_t, PART>(a, grid, L);
    return hipGetLastError();
}

template <int KK, int PK, bool PART>
hipError_t launch_sweep(int b, const SweepArgs &a, int cfg, bool wide, uint64_t grid, const Launch &L) {
    switch (b) {
        case 1: return launch_sweep_b<1, KK, PK, PART>(a, cfg, wide, grid, L);
        case 2: return launch_sweep_b<2, KK, PK, PART>(a, cfg, wide, grid, L);
        case 4: return launch_sweep_b<4, KK, PK, PART>(a, cfg, wide, grid, L);
        default: return launch_sweep_b<8, KK, PK, PART>(a, cfg, wide, grid, L);
    }
}

template <int KK>
hipError_t launch_hist(int b, const HistArgs &a, uint32_t blocks, const Launch &L) {
    switch (b) {
        case 1: launch_on(histogram_kernel<1, KK>, dim3(blocks), dim3(kHistBlock), L, a); break;
        case 2: launch_on(histogram_kernel<2, KK>, dim3(blocks), dim3(kHistBlock), L, a); break;
        case 4: launch_on(histogram_kernel<4, KK>, dim3(blocks), dim3(kHistBlock), L, a); break;
        default: launch_on(histogram_kernel<8, KK>, dim3(blocks), dim3(kHistBlock), L, a); break;
    }
    return hipGetLastError();
}

template <int KK>
hipError_t launch_partition_counts(int b, const PartArgs &pa, const Launch &L) {
    const dim3 grid(pa.partitions);
    // timed as one: the count's start and the scan's end
    const Launch first{L.s, L.start, nullptr}, second{L.s, nullptr, L.stop};
    switch (b) {
        case 1: launch_on(partition_count_kernel<1, KK>, grid, dim3(kHistBlock), first, pa); launch_on(partition_scan_kernel<1>, dim3(1), dim3(256), second, pa); break;
        case 2: launch_on(partition_count_kernel<2, KK>, grid, dim3(kHistBlock), first, pa); launch_on(partition_scan_kernel<2>, dim3(1), dim3(256), second, pa); break;
        case 4: launch_on(partition_count_kernel<4, KK>, grid, dim3(kHistBlock), first, pa); launch_on(partition_scan_kernel<4>, dim3(1), dim3(256), second, pa); break;
        default: launch_on(partition_count_kernel<8, KK>, grid, dim3(kHistBlock), first, pa); launch_on(partition_scan_kernel<8>, dim3(1), dim3(256), second, pa); break;
    }
    return hipGetLastError();
}

template <int B, int KK, int PK>
void launch_resident_b(const ResidentArgs &a, uint64_t rows, uint64_t row_len, const Launch &L) {
    // one workgroup per row; the smallest shape that holds the row
    const dim3 grid(static_cast<uint32_t>(rows));
    if (row_len <= 1024)
        launch_on(resident_sort_kernel<B, 4, 256, KK, PK>, grid, dim3(256), L, a);
    else if (row_len <= 4096)
        launch_on(resident_sort_kernel<B, 16, 256, KK, PK>, grid, dim3(256), L, a);
    else
        launch_on(resident_sort_kernel<B, 16, 512, KK, PK>, grid, dim3(512), L, a);
}

template <int KK, int PK>
hipError_t launch_resident(int b, const ResidentArgs &a, uint64_t rows, uint64_t row_len, const Launch &L) {
    switch (b) {
        case 1: launch_resident_b<1, KK, PK>(a, rows, row_len, L); break;
        case 2: launch_resident_b<2, KK, PK>(a, rows, row_len, L); break;
        case 4: launch_resident_b<4, KK, PK>(a, rows, row_len, L); break;
        default: launch_resident_b<8, KK, PK>(a, rows, row_len, L); break;
    }
    return hipGetLastError();
}

// Workgroups of `kernel` that fit on the current GPU at once (compute units x
// the occupancy per unit), queried once per device and kernel and kept, so a
// call under graph capture makes no query.  0 if the runtime cannot tell.
template <typename Kernel>
uint32_t resident_capacity(Kernel kernel, int block) {
    constexpr int kMaxDevices = 64;
    static std::atomic<uint32_t> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    uint32_t c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0) return c;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess || cus <= 0 ||
        per_cu <= 0)
        return 0;
    c = static_cast<uint32_t>(cus) * static_cast<uint32_t>(per_cu);
    cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <int B, int ITEMS, int BLOCK, int PK>
hipError_t launch_row_resident_cfg(const RowResidentArgs &a, const Launch &L) {
    auto kernel = row_resident_kernel<B, ITEMS, BLOCK, PK>;
    const uint32_t cap = resident_capacity(kernel, BLOCK);
    const uint32_t grid = (cap == 0 || cap > a.rows) ? a.rows : cap;
    launch_on(kernel, dim3(grid), dim3(BLOCK), L, a);
    return hipGetLastError();
}

#ifndef LRS_ROW_ITEMS
#define LRS_ROW_ITEMS 8
#endif
template <int B, int PK>
hipError_t launch_row_resident_b(const RowResidentArgs &a, const Launch &L) {
    // the smallest shape that holds the row
    constexpr int I = LRS_ROW_ITEMS;
    static_assert(1024 * I >= 8192, "the largest shape holds a row of 8192");
    if (a.row_len <= 256u * I) return launch_row_resident_cfg<B, I, 256, PK>(a, L);
    if (a.row_len <= 512u * I) return launch_row_resident_cfg<B, I, 512, PK>(a, L);
    return launch_row_resident_cfg<B, I, 1024, PK>(a, L);
}

template <int PK>
hipError_t launch_row_resident(int b, const RowResidentArgs &a, const Launch &L) {
    switch (b) {
        case 1: return launch_row_resident_b<1, PK>(a, L);
        case 2: return launch_row_resident_b<2, PK>(a, L);
        case 4: return launch_row_resident_b<4, PK>(a, L);
        default: return launch_row_resident_b<8, PK>(a, L);
    }
}

}  // namespace lrs
