// lrs_inst_c32_keys.hip -- 32-bit keys under one constant XOR (signed, descending u32), keys only
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyC32, kPayNone, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyC32, kPayNone, true>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_hist<kKeyC32>(int, const HistArgs &, uint32_t, const Launch &);
template hipError_t launch_partition_counts<kKeyC32>(int, const PartArgs &, const Launch &);
template hipError_t launch_resident<kKeyC32, kResNone>(int, const ResidentArgs &, uint64_t, uint64_t, const Launch &);
}  // namespace lrs
