// bwd_variants_bf16.hip — the backward variants over __bf16 rows (see bwd_table.hpp).
#include "bwd_table.hpp"

namespace minorm {
namespace {
const Variant kVariants[] = {MI_BWD_DTYPE_TABLE(__bf16, MI_NORM_BF16, 8, "_bf16")};
}  // namespace
extern const VariantTable kBwdTableBF16 = {kVariants, (int)(sizeof(kVariants) / sizeof(kVariants[0]))};
}  // namespace minorm
