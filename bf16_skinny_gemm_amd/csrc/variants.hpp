// Compiled variants of the skinny GEMM kernels: the plan fields that select a
// template instance of kernels.hpp, one kernel per token count M.
//
// The variant tables are split over several translation units (variants_*.hip)
// that are compiled in parallel; each instantiates only its own kernels, and the
// host side (skinny_gemm.hip) joins the tables on first use.
#pragma once

#include "skinny_gemm.h"

#include "kernels.hpp"
#include "validate.hpp"

namespace skg_host {

// A compiled variant: the plan fields that select template instances, one
// kernel per M (NULL where that M would not fit the register budget, or for the
// MFMA family beyond M = 4, the rows of its A operand).
struct Variant {
    skinny_plan_t plan;    // threads_per_block / grid_blocks: defaults only
    const void *fn[kMaxM];
    int k_fixed;           // FIXED_K: the only K it computes
    int rows_per_group;    // rows one wave group covers per tile
};

// Register budget per lane, so that no instance spills: x in registers takes
// 4*M*CH VGPRs (at most 128), the weight sets in flight 4*R*CH each (two with
// tile prefetch, one without or with rolling prefetch), the sums M*R; with x in
// registers the three may hold 200 between them (the only instances above that,
// M = 8 with two sets of 2 rows x 4 chunks, spilled). Reading x from LDS one
// chunk ahead (XL = 2) holds 4*M more and is built for M >= 2 only: at M = 1 a
// register copy of x is cheaper.
constexpr bool fits(int M, int CH, int R, int XL, int PF)
{
    const int w = (PF == 1 ? 2 : 1) * R * CH;
    if (XL == 2)
        return M >= 2 && w <= 20;
    return XL ? w <= 20 : (M * CH <= 32 && 4 * (M * CH + w) + M * R <= 200);
}

template <int M, int LPR, int CH, int R, int KW, int XL, bool NT, int PF>
constexpr const void *fixed_fn()
{
    if constexpr (fits(M, CH, R, XL, PF))
        return reinterpret_cast<const void *>(&skg::fixed_k_kernel<M, LPR, CH, R, KW, XL, NT, PF>);
    else
        return nullptr;
}

template <int LPR, int CH, int R, int KW, int XL, bool NT, int PF>
Variant fixed_variant()
{
    Variant v{};
    v.plan = skinny_plan_t{SKINNY_KIND_FIXED_K, 256, LPR, CH, R, KW, NT ? 1 : 0, 0, XL, PF};
    v.fn[0] = fixed_fn<1, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[1] = fixed_fn<2, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[2] = fixed_fn<3, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[3] = fixed_fn<4, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[4] = fixed_fn<5, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[5] = fixed_fn<6, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[6] = fixed_fn<7, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[7] = fixed_fn<8, LPR, CH, R, KW, XL, NT, PF>();
    v.k_fixed = KW * LPR * 8 * CH;
    v.rows_per_group = R * (64 / LPR);
    return v;
}

template <int U, int R, bool NT>
Variant loop_variant()
{
    Variant v{};
    v.plan = skinny_plan_t{SKINNY_KIND_LOOP_K, 256, 64, U, R, 1, NT ? 1 : 0, 0, 1, 0};
    v.fn[0] = reinterpret_cast<const void *>(&skg::loop_k_kernel<1, U, R, NT>);
    v.fn[1] = reinterpret_cast<const void *>(&skg::loop_k_kernel<2, U, R, NT>);
    v.fn[2] = reinterpret_cast<const void *>(&skg::loop_k_kernel<3, U, R, NT>);
    v.fn[3] = reinterpret_cast<const void *>(&skg::loop_k_kernel<4, U, R, NT>);
    v.fn[4] = reinterpret_cast<const void *>(&skg::loop_k_kernel<5, U, R, NT>);
    v.fn[5] = reinterpret_cast<const void *>(&skg::loop_k_kernel<6, U, R, NT>);
    v.fn[6] = reinterpret_cast<const void *>(&skg::loop_k_kernel<7, U, R, NT>);
    v.fn[7] = reinterpret_cast<const void *>(&skg::loop_k_kernel<8, U, R, NT>);
    v.k_fixed = 0;
    v.rows_per_group = R;
    return v;
}

template <int U, int R, int KW, bool PF>
Variant mfma_variant()
{
    Variant v{};
    const int tpb = 64 * (KW > 4 ? KW : 4);
    v.plan = skinny_plan_t{SKINNY_KIND_MFMA, tpb, 16, U, R, KW, 1, 0, 1, PF ? 1 : 0};
    v.fn[0] = reinterpret_cast<const void *>(&skg::mfma_kernel<1, U, R, KW, true, PF>);
    v.fn[1] = reinterpret_cast<const void *>(&skg::mfma_kernel<2, U, R, KW, true, PF>);
    v.fn[2] = reinterpret_cast<const void *>(&skg::mfma_kernel<3, U, R, KW, true, PF>);
    v.fn[3] = reinterpret_cast<const void *>(&skg::mfma_kernel<4, U, R, KW, true, PF>);
    v.k_fixed = 0;
    v.rows_per_group = 4 * R;
    return v;
}

inline Variant scalar_variant()
{
    Variant v{};
    v.plan = skinny_plan_t{SKINNY_KIND_SCALAR, 256, 64, 1, 1, 1, 0, 0, 0, 0};
    v.fn[0] = reinterpret_cast<const void *>(&skg::scalar_kernel<1>);
    v.fn[1] = reinterpret_cast<const void *>(&skg::scalar_kernel<2>);
    v.fn[2] = reinterpret_cast<const void *>(&skg::scalar_kernel<3>);
    v.fn[3] = reinterpret_cast<const void *>(&skg::scalar_kernel<4>);
    v.fn[4] = reinterpret_cast<const void *>(&skg::scalar_kernel<5>);
    v.fn[5] = reinterpret_cast<const void *>(&skg::scalar_kernel<6>);
    v.fn[6] = reinterpret_cast<const void *>(&skg::scalar_kernel<7>);
    v.fn[7] = reinterpret_cast<const void *>(&skg::scalar_kernel<8>);
    v.k_fixed = 0;
    v.rows_per_group = 1;
    return v;
}

// Per (lanes_per_row, chunks, k_split): one or two rows per wave, x in registers
// or LDS, each prefetch mode (none, tile, rolling), all with the non-temporal
// hint; x in LDS read one chunk ahead at one row per wave; plus the plain-cached
// form at one row per wave (the hint won every cell of the gfx950 sweep).
#define SKG_FIXED_XP(LPR, CH, KW, XL, PF)                                                          \
    fixed_variant<LPR, CH, 1, KW, XL, true, PF>(), fixed_variant<LPR, CH, 2, KW, XL, true, PF>()
#define SKG_FIXED(LPR, CH, KW)                                                                      \
    SKG_FIXED_XP(LPR, CH, KW, 0, 0), SKG_FIXED_XP(LPR, CH, KW, 0, 1),                               \
        SKG_FIXED_XP(LPR, CH, KW, 0, 2), SKG_FIXED_XP(LPR, CH, KW, 1, 0),                           \
        SKG_FIXED_XP(LPR, CH, KW, 1, 1), SKG_FIXED_XP(LPR, CH, KW, 1, 2),                           \
        fixed_variant<LPR, CH, 1, KW, 2, true, 0>(), fixed_variant<LPR, CH, 1, KW, 2, true, 1>(),   \
        fixed_variant<LPR, CH, 1, KW, 2, true, 2>(), fixed_variant<LPR, CH, 1, KW, 0, false, 1>()
#define SKG_LOOP(U, R) loop_variant<U, R, false>(), loop_variant<U, R, true>()
#define SKG_MFMA_PF(U, R, KW) mfma_variant<U, R, KW, false>(), mfma_variant<U, R, KW, true>()
#define SKG_MFMA(U, R) SKG_MFMA_PF(U, R, 1), SKG_MFMA_PF(U, R, 2), SKG_MFMA_PF(U, R, 4), SKG_MFMA_PF(U, R, 8)

// One part of the compiled set (a static array owned by its translation unit).
struct VariantSpan {
    const Variant *v;
    int n;
};

// FIXED_K triples (lanes_per_row, chunks, k_split) covering the K of the decode
// projections: 128 (paired f_b/g_b), 1024 and 1536 / 4096 / 8192.
VariantSpan variants_fixed_small();
VariantSpan variants_fixed_k4096();
VariantSpan variants_fixed_k8192();
// LOOP_K (any K % 8 == 0), MFMA (K % (128 * k_split * chunks) == 0) and the
// element-wise SCALAR variant (any K, any alignment; always last).
VariantSpan variants_other();

}  // namespace skg_host
