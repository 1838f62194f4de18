// Row-kernel instances for float16 inputs.
#include "adq_row_impl.h"

namespace adq {
ADQ_DEFINE_ROW_ENTRY(kF16, f16)
}  // namespace adq
