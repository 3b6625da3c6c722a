// fa_fwd_f32_d64.hip - the fp32 forward variants at head dim 64: every
// mask kind, causal or not, with and without dropout.
#include "fa_fwd_f32.h"

namespace fa {

// Host-only accessors (see fa_fwd_bf16_d64.hip).
const Variant* variants_f32_d64(int* n)
{
    static const Variant table[] = {FA_F32_FOR_D_CFG(64, FA_F32_D64_CFG)};
    *n = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

const Variant* variants_f32_dropout_d64(int* n)
{
    static const Variant table[] = {FA_F32_DROP_FOR_D_CFG(64, FA_F32_D64_CFG)};
    *n = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
