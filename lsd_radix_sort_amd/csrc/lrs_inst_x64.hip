// lrs_inst_x64.hip -- other 64-bit keys (signed, double, descending u64), keys only or with a u32 payload
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyX64, kPayNone, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyX64, kPayU32, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_hist<kKeyX64>(int, const HistArgs &, uint32_t, const Launch &);
}  // namespace lrs
