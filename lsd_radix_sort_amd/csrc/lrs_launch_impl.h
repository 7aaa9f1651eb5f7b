// lrs_launch_impl.h -- definitions of the launcher templates declared in
// lrs_launch.h; included only by the lrs_inst_*.hip files, which instantiate
// them (and so compile the kernels) for one key kind each.
#pragma once

#include "lrs_launch.h"

namespace lrs {

template <int B, int ITEMS, int BLOCK, int KK, int PK, typename W, bool PART>
void launch_sweep_cfg(const SweepArgs &a, uint64_t grid_size, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(grid_size));
    sweep_kernel<B, ITEMS, BLOCK, KK, PK, W, PART><<<grid, BLOCK, 0, s>>>(a);
}

template <int B, int KK, int PK, bool PART>
hipError_t launch_sweep_b(const SweepArgs &a, int cfg, bool wide, uint64_t grid, hipStream_t s) {
    constexpr bool k64 = sizeof(typename KeyTraits<KK>::Stored) == 8;
    constexpr TileCfg c0 = tile_cfg_of(k64, 0), c1 = tile_cfg_of(k64, 1), c2 = tile_cfg_of(k64, 2);
    // 64-bit look-back words (and 64-bit store addressing) only occur for rows
    // of 2^29 or more elements (2^30 for 4-byte keys), which always take the
    // largest tile.
    if (wide)
        launch_sweep_cfg<B, c2.items, c2.block, KK, PK, uint64_t, PART>(a, grid, s);
    else if (cfg == 2)
        launch_sweep_cfg<B, c2.items, c2.block, KK, PK, uint32_t, PART>(a, grid, s);
    else if (cfg == 1)
        launch_sweep_cfg<B, c1.items, c1.block, KK, PK, uint32_t, PART>(a, grid, s);
    else
        launch_sweep_cfg<B, c0.items, c0.block, KK, PK, uint32_t, PART>(a, grid, s);
    return hipGetLastError();
}

template <int KK, int PK, bool PART>
hipError_t launch_sweep(int b, const SweepArgs &a, int cfg, bool wide, uint64_t grid, hipStream_t s) {
    switch (b) {
        case 1: return launch_sweep_b<1, KK, PK, PART>(a, cfg, wide, grid, s);
        case 2: return launch_sweep_b<2, KK, PK, PART>(a, cfg, wide, grid, s);
        case 4: return launch_sweep_b<4, KK, PK, PART>(a, cfg, wide, grid, s);
        default: return launch_sweep_b<8, KK, PK, PART>(a, cfg, wide, grid, s);
    }
}

template <int KK>
hipError_t launch_hist(int b, const HistArgs &a, uint32_t blocks, hipStream_t s) {
    switch (b) {
        case 1: histogram_kernel<1, KK><<<blocks, kHistBlock, 0, s>>>(a); break;
        case 2: histogram_kernel<2, KK><<<blocks, kHistBlock, 0, s>>>(a); break;
        case 4: histogram_kernel<4, KK><<<blocks, kHistBlock, 0, s>>>(a); break;
        default: histogram_kernel<8, KK><<<blocks, kHistBlock, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

template <int KK>
hipError_t launch_partition_counts(int b, const PartArgs &pa, hipStream_t s) {
    const dim3 grid(pa.partitions);
    switch (b) {
        case 1: partition_count_kernel<1, KK><<<grid, kHistBlock, 0, s>>>(pa); partition_scan_kernel<1><<<1, 256, 0, s>>>(pa); break;
        case 2: partition_count_kernel<2, KK><<<grid, kHistBlock, 0, s>>>(pa); partition_scan_kernel<2><<<1, 256, 0, s>>>(pa); break;
        case 4: partition_count_kernel<4, KK><<<grid, kHistBlock, 0, s>>>(pa); partition_scan_kernel<4><<<1, 256, 0, s>>>(pa); break;
        default: partition_count_kernel<8, KK><<<grid, kHistBlock, 0, s>>>(pa); partition_scan_kernel<8><<<1, 256, 0, s>>>(pa); break;
    }
    return hipGetLastError();
}

template <int B, int KK, int PK>
void launch_resident_b(const ResidentArgs &a, uint64_t rows, uint64_t row_len, hipStream_t s) {
    // one workgroup per row; the smallest shape that holds the row
    const dim3 grid(static_cast<uint32_t>(rows));
    if (row_len <= 1024)
        resident_sort_kernel<B, 4, 256, KK, PK><<<grid, 256, 0, s>>>(a);
    else if (row_len <= 4096)
        resident_sort_kernel<B, 16, 256, KK, PK><<<grid, 256, 0, s>>>(a);
    else
        resident_sort_kernel<B, 16, 512, KK, PK><<<grid, 512, 0, s>>>(a);
}

template <int KK, int PK>
hipError_t launch_resident(int b, const ResidentArgs &a, uint64_t rows, uint64_t row_len, hipStream_t s) {
    switch (b) {
        case 1: launch_resident_b<1, KK, PK>(a, rows, row_len, s); break;
        case 2: launch_resident_b<2, KK, PK>(a, rows, row_len, s); break;
        case 4: launch_resident_b<4, KK, PK>(a, rows, row_len, s); break;
        default: launch_resident_b<8, KK, PK>(a, rows, row_len, s); break;
    }
    return hipGetLastError();
}

}  // namespace lrs
