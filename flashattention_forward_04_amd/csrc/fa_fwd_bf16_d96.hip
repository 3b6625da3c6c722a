// fa_fwd_bf16_d96.hip - the bf16 forward variants at head dim 96: every
// mask kind, causal or not, with and without dropout.
#include "fa_fwd_bf16.h"

namespace fa {

// Host-only accessors: a namespace-scope const table would also be emitted
// for the device, where the launch functions do not exist.
const Variant* variants_bf16_d96(int* n)
{
    static const Variant table[] = {FA_BF16_FOR_D(96, FA_BF16_D96_CFG, FA_BF16_D96_MASKED_CFG)};
    *n = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

const Variant* variants_bf16_dropout_d96(int* n)
{
    static const Variant table[] = {FA_BF16_DROP_FOR_D(96, FA_BF16_D96_CFG, FA_BF16_D96_MASKED_CFG)};
    *n = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
