// lrs_inst_rows_packed.hip -- the last pass of a row sort whose elements travel
// as packed words (key << 16 | column): words in, pattern and int64 column out
// (the kernels of one key kind, compiled in their own translation unit).
#include "lrs_launch_impl.h"

namespace lrs {

template hipError_t launch_sweep<kKeyU32, kPayUnpackLast, false>(int, const SweepArgs &, int, bool, uint64_t, const Launch &);

}  // namespace lrs
