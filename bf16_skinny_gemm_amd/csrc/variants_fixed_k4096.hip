// FIXED_K variants for K = 4096.
#include "variants.hpp"

namespace skg_host {

VariantSpan variants_fixed_k4096()
{
    static const Variant v[] = {
        SKG_FIXED(64, 8, 1), SKG_FIXED(64, 4, 2), SKG_FIXED(64, 2, 4),
    };
    return VariantSpan{v, (int)(sizeof(v) / sizeof(v[0]))};
}

}  // namespace skg_host
