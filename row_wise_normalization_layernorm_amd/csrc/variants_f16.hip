// variants_f16.hip — the kernel variants over _Float16 rows (see variant_table.hpp).
#include "variant_table.hpp"

namespace minorm {
namespace {
const Variant kVariants[] = {MI_DTYPE_TABLE(_Float16, MI_NORM_F16, 8, "_f16")};
}  // namespace
extern const VariantTable kTableF16 = {kVariants, (int)(sizeof(kVariants) / sizeof(kVariants[0]))};
}  // namespace minorm
