// libtq: decode kernels for fp32 activations quantised to int8 in the kernel,
// up to 8 tokens per launch (all scale layouts, K = 1..4).
#include "tq_gemv_impl.h"

namespace tqk {
const single_fn* single_table_3_2() { return TablesFor<3, 8>::single; }
const grouped_fn* grouped_table_3_2() { return TablesFor<3, 8>::grouped; }
}  // namespace tqk
