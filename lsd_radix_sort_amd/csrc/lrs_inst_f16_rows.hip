// lrs_inst_f16_rows.hip -- fp16/bf16 row sort with the column index as payload
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyF16, kPayIdxFirst, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyF16, kPayU32, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyF16, kPayIdxLast, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_sweep<kKeyF16, kPayPackFirst, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);
template hipError_t launch_hist<kKeyF16>(int, const HistArgs &, uint32_t, const Launch &);
template hipError_t launch_row_resident<kResIndex>(int, const RowResidentArgs &, const Launch &);
template hipError_t launch_row_resident<kResU32>(int, const RowResidentArgs &, const Launch &);
}  // namespace lrs
