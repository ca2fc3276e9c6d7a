// LOOP_K, MFMA and SCALAR variants.
#include "variants.hpp"

namespace skg_host {

VariantSpan variants_other()
{
    static const Variant v[] = {
        // any K % 8 == 0
        SKG_LOOP(2, 1), SKG_LOOP(4, 1), SKG_LOOP(8, 1), SKG_LOOP(2, 2), SKG_LOOP(4, 2),
        // matrix cores: K % (128 * k_split * chunks) == 0
        SKG_MFMA(1, 1), SKG_MFMA(2, 1), SKG_MFMA(4, 1), SKG_MFMA(8, 1), SKG_MFMA(2, 2),
        SKG_MFMA(4, 2),
        // any K, any alignment (kept last)
        scalar_variant(),
    };
    return VariantSpan{v, (int)(sizeof(v) / sizeof(v[0]))};
}

}  // namespace skg_host
