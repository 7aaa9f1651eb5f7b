// lrs_inst_u32_keys.hip -- u32 keys, keys only: sweep (both scan strategies), histogram, partition counts, resident sort
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyU32, kPayNone, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyU32, kPayNone, true>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_hist<kKeyU32>(int, const HistArgs &, uint32_t, const Launch &);
template hipError_t launch_partition_counts<kKeyU32>(int, const PartArgs &, const Launch &);
template hipError_t launch_resident<kKeyU32, kResNone>(int, const ResidentArgs &, uint64_t, uint64_t, const Launch &);
}  // namespace lrs
