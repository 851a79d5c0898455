// bwd_variants_f32.hip — the backward variants over float rows (see bwd_table.hpp).
#include "bwd_table.hpp"

namespace minorm {
namespace {
const Variant kVariants[] = {MI_BWD_DTYPE_TABLE(float, MI_NORM_F32, 4, "")};
}  // namespace
extern const VariantTable kBwdTableF32 = {kVariants, (int)(sizeof(kVariants) / sizeof(kVariants[0]))};
}  // namespace minorm
