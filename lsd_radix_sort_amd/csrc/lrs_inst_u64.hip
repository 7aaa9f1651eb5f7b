// lrs_inst_u64.hip -- u64 keys, keys only or with a u32 payload
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyU64, kPayNone, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyU64, kPayU32, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_hist<kKeyU64>(int, const HistArgs &, uint32_t, const Launch &);
}  // namespace lrs
