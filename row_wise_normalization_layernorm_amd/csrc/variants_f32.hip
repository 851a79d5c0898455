// variants_f32.hip — the kernel variants over float rows (see variant_table.hpp).
#include "variant_table.hpp"

namespace minorm {
namespace {
const Variant kVariants[] = {MI_DTYPE_TABLE(float, MI_NORM_F32, 4, "")};
}  // namespace
extern const VariantTable kTableF32 = {kVariants, (int)(sizeof(kVariants) / sizeof(kVariants[0]))};
}  // namespace minorm
