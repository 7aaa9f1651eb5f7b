// lrs_inst_u32_pairs.hip -- u32 keys with a u32 payload: sweep (both scan strategies), resident sort
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyU32, kPayU32, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyU32, kPayU32, true>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_resident<kKeyU32, kResU32>(int, const ResidentArgs &, uint64_t, uint64_t, const Launch &);
}  // namespace lrs
