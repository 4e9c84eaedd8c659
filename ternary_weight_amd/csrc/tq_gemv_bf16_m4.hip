// libtq: decode kernels for bf16 activations, up to 4 token(s) per launch
// (all scale layouts, K = 1..4).
#include "tq_gemv_impl.h"

namespace tqk {
const single_fn* single_table_1_1() { return TablesFor<1, 4>::single; }
const grouped_fn* grouped_table_1_1() { return TablesFor<1, 4>::grouped; }
const wave_items_fn* wave_table_1_1() { return TablesFor<1, 4>::wave; }
}  // namespace tqk
