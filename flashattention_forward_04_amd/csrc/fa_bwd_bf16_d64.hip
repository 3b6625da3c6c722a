// fa_bwd_bf16_d64.hip - the bf16 backward variants at head dim 64: every
// mask kind, causal or not.
#include "fa_bwd_bf16.h"

namespace fa {

// Host-only accessor (a namespace-scope table would also be emitted for the
// device, where the launch functions do not exist).
const BwdVariant* bwd_variants_bf16_d64(int* n)
{
    static const BwdVariant table[] = {FA_BWD_FOR_D(64, FA_BWD_D64_CFG)};
    *n = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fa
