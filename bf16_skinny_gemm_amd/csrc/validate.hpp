// Host-side argument checks of the C ABI (include/skinny_gemm.h): plain C++ with
// no HIP code, so that a sanitizer build on the CPU (g++ -fsanitize=address,
// undefined) exercises exactly the checks the library runs before any launch.
#pragma once

#include <cstddef>
#include <cstdint>

#include "skinny_gemm.h"

namespace skg_host {

// Largest token count M the kernels are compiled for.
constexpr int kMaxM = 8;

inline bool overlaps(const void *a, size_t la, const void *b, size_t lb)
{
    if (!a || !b || la == 0 || lb == 0)
        return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + lb && pb < pa + la;
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Call {
    const void *x, *x1;  // x of W0 and of W1 (x1 == x for the shared-input pair)
    const void *w0, *w1;
    void *y0, *y1;
    int M, N, K, nmats;
    int ldx, ldy;        // row strides of x/x1 and y0/y1, in elements
    int out_f32;         // 1: float32 outputs, 0: bfloat16
};

inline Call single_call(const void *x, const void *W, void *y, int M, int N, int K, int out_f32)
{
    return Call{x, x, W, nullptr, y, nullptr, M, N, K, 1, K, N, out_f32};
}

// Bytes spanned by `rows` rows of `width` elements at `stride` elements.
inline size_t span(int rows, int width, int stride, size_t elem)
{
    return rows > 0 && width > 0 ? ((size_t)(rows - 1) * stride + width) * elem : 0;
}

// Two same-shape row-strided blocks (rows x width at the same stride, in bytes)
// share no byte. Exact when the strides are equal: the second block's rows must
// fall in the gaps between the first block's rows, or the spans must not meet.
inline bool strided_disjoint(const void *p, const void *q, int rows, size_t width, size_t stride)
{
    const size_t s = (size_t)(rows - 1) * stride + width;
    if (!overlaps(p, s, q, s))
        return true;
    const long long d = (long long)(reinterpret_cast<uintptr_t>(q) - reinterpret_cast<uintptr_t>(p));
    const long long st = (long long)stride;
    const long long r = ((d % st) + st) % st;  // q's rows start r bytes into p's stride period
    return r >= (long long)width && r + (long long)width <= st;
}

inline int validate(const Call &c)
{
    if (c.M < 0 || c.M > kMaxM || c.N < 0 || c.K < 0)
        return SKINNY_ERR_INVALID_ARG;
    if (c.M == 0 || c.N == 0)
        return SKINNY_OK;
    if (c.ldx < c.K || c.ldy < c.N)
        return SKINNY_ERR_INVALID_ARG;
    if (!c.y0 || (c.nmats == 2 && !c.y1))
        return SKINNY_ERR_INVALID_ARG;
    if (c.K > 0 && (!c.x || !c.w0 || (c.nmats == 2 && (!c.w1 || !c.x1))))
        return SKINNY_ERR_INVALID_ARG;
    const void *ptrs[6] = {c.x, c.nmats == 2 ? c.x1 : nullptr, c.w0, c.nmats == 2 ? c.w1 : nullptr,
                           c.y0, c.nmats == 2 ? c.y1 : nullptr};
    for (const void *p : ptrs)
        if (p && !aligned(p, 2))
            return SKINNY_ERR_INVALID_ARG;
    const size_t ye = c.out_f32 ? 4 : 2;
    if (c.out_f32 && (!aligned(c.y0, 4) || (c.nmats == 2 && !aligned(c.y1, 4))))
        return SKINNY_ERR_INVALID_ARG;
    const size_t xb = span(c.M, c.K, c.ldx, 2), wb = (size_t)c.N * c.K * 2;
    const size_t yb = span(c.M, c.N, c.ldy, ye);
    for (int i = 0; i < c.nmats; ++i) {
        void *y = i ? c.y1 : c.y0;
        if (overlaps(y, yb, c.x, xb) || overlaps(y, yb, c.w0, wb) ||
            (c.nmats == 2 && (overlaps(y, yb, c.w1, wb) || overlaps(y, yb, c.x1, xb))))
            return SKINNY_ERR_INVALID_ARG;
    }
    if (c.nmats == 2 && !strided_disjoint(c.y0, c.y1, c.M, (size_t)c.N * ye, (size_t)c.ldy * ye))
        return SKINNY_ERR_INVALID_ARG;
    return SKINNY_OK;
}

// 128-bit loads need 16-byte aligned rows of x and W; buffer offsets are 32-bit.
inline bool vector_ok(const Call &c)
{
    const bool al = aligned(c.x, 16) && aligned(c.w0, 16) &&
                    (c.nmats == 1 || (aligned(c.w1, 16) && aligned(c.x1, 16)));
    return al && c.K % 8 == 0 && c.ldx % 8 == 0 && c.K <= (1 << 20) &&
           span(c.M, c.K, c.ldx, 2) < (1u << 31);
}

// The M output rows of y (M - 1 row strides plus N elements), which the vector
// kernels store through as one buffer resource, must fit in 31 bits of bytes.
inline bool out_span_ok(const Call &c)
{
    return ((long long)(c.M - 1) * c.ldy + c.N) * (c.out_f32 ? 4 : 2) <= 0x7FFFFFFFLL;
}

// Key of a default-plan call in the resolved-launch cache: bit 63 set (so never
// 0, an empty slot, or 1, a slot being written), device (6 bits),
// nmats - 1 (1), M - 1 (3), K (21: K <= 2^20 on the vector path), N (31).
inline uint64_t cache_key(int dev, const Call &c)
{
    return (1ull << 63) | ((uint64_t)dev << 56) | ((uint64_t)(c.nmats - 1) << 55) |
           ((uint64_t)(c.M - 1) << 52) | ((uint64_t)c.K << 31) | (uint64_t)c.N;
}

// ---- cross-block split-K (split_k.hip): the checks and the workspace layout ----

// Largest block of the split-K kernels, in threads (8 waves).
constexpr int kSplitMaxThreads = 512;
// Workspace layout, the same for every call: kSplitCountWords 32-bit arrival
// counters (tile t uses word t) in the first 64 KiB, then the float partials
// [S][M][N]. Counters stay at zero between calls and no call writes partials over
// them, so one workspace serves calls of any shape it is large enough for.
constexpr size_t kSplitCountWords = 16384;
constexpr size_t kSplitPartOffset = kSplitCountWords * 4;

struct SplitLayout {
    size_t part_bytes, total;
    long long tiles;
};

// Row tiles and workspace bytes of a call: tiles of (threads / 64) * rows_per_group
// rows, S * M * N float partials after the counters.
inline SplitLayout split_layout(int threads, int rows_per_group, int S, int M, int N)
{
    SplitLayout l{};
    const long long rows_t = (long long)(threads / 64) * rows_per_group;
    l.tiles = ((long long)N + rows_t - 1) / rows_t;
    l.part_bytes = (size_t)S * (size_t)M * (size_t)N * 4;
    l.total = kSplitPartOffset + l.part_bytes;
    return l;
}

// The plan fields a split-K plan must hold, apart from which variant it names and
// whether its slices make K (the caller checks those against the compiled set).
inline bool split_fields_ok(const skinny_plan_t &p)
{
    const int t = p.threads_per_block;
    return p.kind == SKINNY_KIND_SPLIT_K && t >= 64 && t <= kSplitMaxThreads && t % 64 == 0 &&
           p.k_split >= 1 && p.k_split <= 64 && p.nontemporal == 1 && p.grid_blocks == 0 &&
           p.x_in_lds == 0 && p.prefetch == 0;
}

// A split-K call beyond validate(): K > 0 and the vector path's conditions (there
// is no element-wise split-K kernel).
inline bool split_call_ok(const Call &c) { return c.K > 0 && vector_ok(c) && out_span_ok(c); }

// The layout fits the counters, and every block and wave index stays inside int.
inline bool split_layout_ok(const SplitLayout &l, int S)
{
    return l.tiles >= 1 && (size_t)l.tiles <= kSplitCountWords && l.tiles * (long long)S <= 0x7FFFFFFFLL;
}

// A caller's workspace: present, 256-byte aligned, large enough for the layout and
// sharing no byte with x, W or y.
inline bool split_workspace_ok(const Call &c, const void *ws, size_t bytes, const SplitLayout &l)
{
    if (!ws || !aligned(ws, 256) || bytes < l.total)
        return false;
    const size_t xb = span(c.M, c.K, c.ldx, 2), wb = (size_t)c.N * c.K * 2;
    const size_t yb = span(c.M, c.N, c.ldy, c.out_f32 ? 4 : 2);
    return !overlaps(ws, l.total, c.x, xb) && !overlaps(ws, l.total, c.w0, wb) && !overlaps(ws, l.total, c.y0, yb);
}

// Looks up device `dev`'s copy of the allocation-free split-K entry point's static
// workspace (split_k.hip), with that device made current for the lookup and the
// caller's device restored; called by skinny_gemm_init. Returns a status code.
int split_k_scratch_setup(int dev);

}  // namespace skg_host
