// libtq: decode kernels for i8 activations, up to 16 token(s) per launch
// (all scale layouts, K = 1..4).
#include "tq_gemv_impl.h"

namespace tqk {
const single_fn* single_table_2_2() { return TablesFor<2, 16>::single; }
const grouped_fn* grouped_table_2_2() { return TablesFor<2, 16>::grouped; }
}  // namespace tqk
