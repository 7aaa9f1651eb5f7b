// lrs_inst_c32_pairs.hip -- 32-bit keys under one constant XOR (signed, descending u32) with a u32 payload
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyC32, kPayU32, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyC32, kPayU32, true>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_resident<kKeyC32, kResU32>(int, const ResidentArgs &, uint64_t, uint64_t, const Launch &);
}  // namespace lrs
