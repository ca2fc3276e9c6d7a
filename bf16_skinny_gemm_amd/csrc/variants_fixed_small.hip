// FIXED_K variants for K = 128 (paired f_b/g_b), 1024 and 1536.
#include "variants.hpp"

namespace skg_host {

VariantSpan variants_fixed_small()
{
    static const Variant v[] = {
        // K = 128
        SKG_FIXED(16, 1, 1), SKG_FIXED(8, 2, 1),
        // K = 1024
        SKG_FIXED(64, 2, 1), SKG_FIXED(32, 4, 1), SKG_FIXED(64, 1, 2),
        // K = 1536
        SKG_FIXED(64, 3, 1), SKG_FIXED(32, 3, 2),
    };
    return VariantSpan{v, (int)(sizeof(v) / sizeof(v[0]))};
}

}  // namespace skg_host
