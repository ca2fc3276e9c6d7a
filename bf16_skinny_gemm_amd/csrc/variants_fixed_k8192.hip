// FIXED_K variants for K = 8192.
#include "variants.hpp"

namespace skg_host {

VariantSpan variants_fixed_k8192()
{
    static const Variant v[] = {
        SKG_FIXED(64, 16, 1), SKG_FIXED(64, 8, 2), SKG_FIXED(64, 4, 4),
    };
    return VariantSpan{v, (int)(sizeof(v) / sizeof(v[0]))};
}

}  // namespace skg_host
