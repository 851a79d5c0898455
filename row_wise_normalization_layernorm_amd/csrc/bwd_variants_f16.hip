// bwd_variants_f16.hip — the backward variants over _Float16 rows (see bwd_table.hpp).
#include "bwd_table.hpp"

namespace minorm {
namespace {
const Variant kVariants[] = {MI_BWD_DTYPE_TABLE(_Float16, MI_NORM_F16, 8, "_f16")};
}  // namespace
extern const VariantTable kBwdTableF16 = {kVariants, (int)(sizeof(kVariants) / sizeof(kVariants[0]))};
}  // namespace minorm
