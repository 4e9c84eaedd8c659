// libtq: decode kernels for f32 activations, up to 1 token(s) per launch
// (all scale layouts, K = 1..4).
#include "tq_gemv_impl.h"

namespace tqk {
const single_fn* single_table_0_0() { return TablesFor<0, 1>::single; }
const grouped_fn* grouped_table_0_0() { return TablesFor<0, 1>::grouped; }
}  // namespace tqk
