// lrs_inst_x32_pairs.hip -- 32-bit keys under the two-mask transform (floats) with a u32 payload
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyX32, kPayU32, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyX32, kPayU32, true>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_resident<kKeyX32, kResU32>(int, const ResidentArgs &, uint64_t, uint64_t, const Launch &);
}  // namespace lrs
