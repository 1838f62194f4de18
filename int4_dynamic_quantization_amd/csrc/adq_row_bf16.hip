// Row-kernel instances for bfloat16 inputs.
#include "adq_row_impl.h"

namespace adq {
ADQ_DEFINE_ROW_ENTRY(kBF16, bf16)
}  // namespace adq
