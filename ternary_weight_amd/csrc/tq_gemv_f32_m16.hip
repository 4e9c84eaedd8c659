// libtq: decode kernels for f32 activations, up to 16 token(s) per launch
// (all scale layouts, K = 1..4).
#include "tq_gemv_impl.h"

namespace tqk {
const single_fn* single_table_0_2() { return TablesFor<0, 16>::single; }
const grouped_fn* grouped_table_0_2() { return TablesFor<0, 16>::grouped; }
}  // namespace tqk
