// fa_fwd_f32_d80.hip - the fp32 forward variants at head dim 80: every
// mask kind, causal or not, with and without dropout.
#include "fa_fwd_f32.h"

namespace fa {

// Host-only accessors (see fa_fwd_bf16_d80.hip).
const Variant* variants_f32_d80(int* n)
{
    static const Variant table[] = {FA_F32_FOR_D_CFG(80, FA_F32_D80_CFG)};
    *n = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

const Variant* variants_f32_dropout_d80(int* n)
{
    static const Variant table[] = {FA_F32_DROP_FOR_D_CFG(80, FA_F32_D80_CFG)};
    *n = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
