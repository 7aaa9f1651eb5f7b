// lrs_inst_x32_keys.hip -- 32-bit keys under the two-mask transform (floats), keys only
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyX32, kPayNone, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyX32, kPayNone, true>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_hist<kKeyX32>(int, const HistArgs &, uint32_t, const Launch &);
template hipError_t launch_partition_counts<kKeyX32>(int, const PartArgs &, const Launch &);
template hipError_t launch_resident<kKeyX32, kResNone>(int, const ResidentArgs &, uint64_t, uint64_t, const Launch &);
}  // namespace lrs
