// variants_bf16.hip — the kernel variants over __bf16 rows (see variant_table.hpp).
#include "variant_table.hpp"

namespace minorm {
namespace {
const Variant kVariants[] = {MI_DTYPE_TABLE(__bf16, MI_NORM_BF16, 8, "_bf16")};
}  // namespace
extern const VariantTable kTableBF16 = {kVariants, (int)(sizeof(kVariants) / sizeof(kVariants[0]))};
}  // namespace minorm
