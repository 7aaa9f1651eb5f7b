// lrs_launch.h -- host-side launchers of the sort kernels (internal header).
//
// The launchers are function templates over the key kind and payload kind;
// each lrs_inst_*.hip file instantiates the ones of one key kind, so the
// kernels compile in separate translation units in parallel.  lrs_host.hip
// (the driver and C ABI) sees only these declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrs_dispatch.h"
#include "lrs_kernels.h"

namespace lrs {

// Sweep tile shapes (threads x keys per thread).  Long rows use the largest;
// shorter inputs a smaller one so the grid still has several tiles per CU and
// little of the last tile of each row is padding.
struct TileCfg {
    int block;
    int items;
    uint64_t tile;
};
constexpr TileCfg kTileCfgs[3] = {
    {256, 16, 4096}, {512, 16, 8192}, {kSweepBlock, LRS_SWEEP_ITEMS, uint64_t(kSweepBlock) * LRS_SWEEP_ITEMS}};
// Sweeps of 4-byte words with no payload phase (keys only, and the row-sort
// passes over packed key/column words) hold fewer registers per element: a
// larger largest tile (rows of 65536 then take four tiles instead of eight).
constexpr TileCfg kTileCfgsKeys[3] = {
    {256, 16, 4096}, {512, 16, 8192},
    {kSweepBlock, LRS_SWEEP_KEYS_ITEMS, uint64_t(kSweepBlock) * LRS_SWEEP_KEYS_ITEMS}};
// 64-bit keys take twice the registers and LDS per key: half the keys per tile.
constexpr TileCfg kTileCfgs64[3] = {{256, 8, 2048}, {512, 8, 4096}, {512, 16, 8192}};
constexpr bool no_payload_phase(int pk) { return pk == kPayNone || pk == kPayPackFirst || pk == kPayUnpackLast; }
constexpr TileCfg tile_cfg_of(bool key64, int c, bool keys_only) {
    return key64 ? kTileCfgs64[c] : keys_only ? kTileCfgsKeys[c] : kTileCfgs[c];
}

// One LSD pass: `grid` workgroups (one per tile, or one per partition with
// PART), tile shape `cfg`, 64-bit look-back words and store addresses when
// `wide`.
template <int KK, int PK, bool PART>
hipError_t launch_sweep(int b, const SweepArgs &a, int cfg, bool wide, uint64_t grid, const Launch &L);

// All passes' digit counts in one read of the keys.
template <int KK>
hipError_t launch_hist(int b, const HistArgs &a, uint32_t blocks, const Launch &L);

// Reduce-then-scan: per-partition counts of one pass digit, then their scan.
template <int KK>
hipError_t launch_partition_counts(int b, const PartArgs &pa, const Launch &L);

// Whole-row resident sort, one workgroup per row (32- and 64-bit keys).
template <int KK, int PK>
hipError_t launch_resident(int b, const ResidentArgs &a, uint64_t rows, uint64_t row_len, const Launch &L);

// Whole-row sort of 16-bit float rows: as many workgroups as fit on the GPU at
// once (at most one per row), each looping over rows.
template <int PK>
hipError_t launch_row_resident(int b, const RowResidentArgs &a, const Launch &L);

}  // namespace lrs
