// Host side of libskinny_gemm_bf16.so: compiled variants, the plan table,
// argument validation and the C ABI declared in include/skinny_gemm.h.
//
// Dispatch follows the plan-table design of vLLM PR #65306 (SM90 skinny GEMM
// plans), section Details: a table keyed by architecture and local (N, K), per
// token count M, with a default path for shapes it does not list; rebuilt for
// gfx950: the table holds launch plans of the hand-written kernels in
// kernels.hpp, and a shape missing from it gets a heuristic default plan
// instead of a different library.
#include "skinny_gemm.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "kernels.hpp"

namespace {

constexpr int kVersion = 100;  // 0.1.0

// A compiled variant: the plan fields that select template instances, one
// kernel per M (NULL where that M would not fit the register budget).
struct Variant {
    skinny_plan_t plan;    // threads_per_block / grid_blocks: defaults only
    const void *fn[4];
    int k_fixed;           // FIXED_K: the only K it computes
    int rows_per_group;    // rows one wave group covers per tile
};

// Register budget per lane, so that no instance spills: x in registers takes
// 4*M*CH VGPRs (at most 128), the weight sets in flight 4*R*CH each (two with
// tile prefetch, one without or with rolling prefetch).
constexpr bool fits(int M, int CH, int R, bool XL, int PF)
{
    const int w = (PF == 1 ? 2 : 1) * R * CH;
    return XL ? w <= 20 : (M * CH <= 32 && M * CH + w <= 48);
}

template <int M, int LPR, int CH, int R, int KW, bool XL, bool NT, int PF>
constexpr const void *fixed_fn()
{
    if constexpr (fits(M, CH, R, XL, PF))
        return reinterpret_cast<const void *>(&skg::fixed_k_kernel<M, LPR, CH, R, KW, XL, NT, PF>);
    else
        return nullptr;
}

template <int LPR, int CH, int R, int KW, bool XL, bool NT, int PF>
Variant fixed_variant()
{
    Variant v{};
    v.plan = skinny_plan_t{SKINNY_KIND_FIXED_K, 256, LPR, CH, R, KW, NT ? 1 : 0, 0, XL ? 1 : 0, PF};
    v.fn[0] = fixed_fn<1, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[1] = fixed_fn<2, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[2] = fixed_fn<3, LPR, CH, R, KW, XL, NT, PF>();
    v.fn[3] = fixed_fn<4, LPR, CH, R, KW, XL, NT, PF>();
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

Variant scalar_variant()
{
    Variant v{};
    v.plan = skinny_plan_t{SKINNY_KIND_SCALAR, 256, 64, 1, 1, 1, 0, 0, 0, 0};
    v.fn[0] = reinterpret_cast<const void *>(&skg::scalar_kernel<1>);
    v.fn[1] = reinterpret_cast<const void *>(&skg::scalar_kernel<2>);
    v.fn[2] = reinterpret_cast<const void *>(&skg::scalar_kernel<3>);
    v.fn[3] = reinterpret_cast<const void *>(&skg::scalar_kernel<4>);
    v.k_fixed = 0;
    v.rows_per_group = 1;
    return v;
}

// Per (lanes_per_row, chunks, k_split): one or two rows per wave, x in registers
// or LDS, each prefetch mode (none, tile, rolling), all with the non-temporal
// hint; plus the plain-cached form at one row per wave (the hint won every cell
// of the gfx950 sweep).
#define SKG_FIXED_XP(LPR, CH, KW, XL, PF)                                                          \
    fixed_variant<LPR, CH, 1, KW, XL, true, PF>(), fixed_variant<LPR, CH, 2, KW, XL, true, PF>()
#define SKG_FIXED(LPR, CH, KW)                                                                      \
    SKG_FIXED_XP(LPR, CH, KW, false, 0), SKG_FIXED_XP(LPR, CH, KW, false, 1),                       \
        SKG_FIXED_XP(LPR, CH, KW, false, 2), SKG_FIXED_XP(LPR, CH, KW, true, 0),                    \
        SKG_FIXED_XP(LPR, CH, KW, true, 1), SKG_FIXED_XP(LPR, CH, KW, true, 2),                     \
        fixed_variant<LPR, CH, 1, KW, false, false, 1>()
#define SKG_LOOP(U, R) loop_variant<U, R, false>(), loop_variant<U, R, true>()
#define SKG_MFMA_PF(U, R, KW) mfma_variant<U, R, KW, false>(), mfma_variant<U, R, KW, true>()
#define SKG_MFMA(U, R) SKG_MFMA_PF(U, R, 1), SKG_MFMA_PF(U, R, 2), SKG_MFMA_PF(U, R, 4), SKG_MFMA_PF(U, R, 8)

// The compiled set. FIXED_K triples (lanes_per_row, chunks, k_split) cover the
// K of the decode projections: 128 (paired f_b/g_b), 1024, 1536, 4096, 8192.
const Variant kAllVariants[] = {
    // K = 128
    SKG_FIXED(16, 1, 1), SKG_FIXED(8, 2, 1),
    // K = 1024
    SKG_FIXED(64, 2, 1), SKG_FIXED(32, 4, 1), SKG_FIXED(64, 1, 2),
    // K = 1536
    SKG_FIXED(64, 3, 1), SKG_FIXED(32, 3, 2),
    // K = 4096
    SKG_FIXED(64, 8, 1), SKG_FIXED(64, 4, 2), SKG_FIXED(64, 2, 4),
    // K = 8192
    SKG_FIXED(64, 16, 1), SKG_FIXED(64, 8, 2), SKG_FIXED(64, 4, 4),
    // any K % 8 == 0
    SKG_LOOP(2, 1), SKG_LOOP(4, 1), SKG_LOOP(8, 1), SKG_LOOP(2, 2), SKG_LOOP(4, 2),
    // matrix cores: K % (128 * k_split * chunks) == 0
    SKG_MFMA(1, 1), SKG_MFMA(2, 1), SKG_MFMA(4, 1), SKG_MFMA(8, 1), SKG_MFMA(2, 2), SKG_MFMA(4, 2),
    // any K, any alignment
    scalar_variant(),
};
constexpr int kNumAll = sizeof(kAllVariants) / sizeof(kAllVariants[0]);

// The enumerable set: every entry of kAllVariants that runs at least one M.
struct Registry {
    const Variant *v[kNumAll];
    int n;
    const Variant *scalar;
};

const Registry &registry()
{
    static const Registry r = [] {
        Registry q{};
        for (const Variant &v : kAllVariants) {
            if (v.fn[0] || v.fn[1] || v.fn[2] || v.fn[3])
                q.v[q.n++] = &v;
            if (v.plan.kind == SKINNY_KIND_SCALAR)
                q.scalar = &v;
        }
        return q;
    }();
    return r;
}

// Tuned plans: (N, K, M) -> plan, generated by the on-device sweep.
struct PlanEntry {
    int N, K, M;
    skinny_plan_t plan;
};
const PlanEntry kPlanTable[] = {
#include "plans_gfx950.inc"
    {0, 0, 0, {0, 0, 0, 0, 0, 0, 0, 0, 0, 0}},  // sentinel
};
constexpr int kNumPlans = sizeof(kPlanTable) / sizeof(kPlanTable[0]) - 1;

bool same_variant(const skinny_plan_t &a, const skinny_plan_t &b)
{
    return a.kind == b.kind && a.lanes_per_row == b.lanes_per_row && a.chunks == b.chunks &&
           a.rows_per_wave == b.rows_per_wave && a.k_split == b.k_split &&
           a.nontemporal == b.nontemporal && a.x_in_lds == b.x_in_lds && a.prefetch == b.prefetch;
}

const Variant *find_variant(const skinny_plan_t &p)
{
    const Registry &r = registry();
    for (int i = 0; i < r.n; ++i)
        if (same_variant(r.v[i]->plan, p))
            return r.v[i];
    return nullptr;
}

// Default plan when the table has no entry (for aligned, K % 8 == 0 calls).
skinny_plan_t default_plan(int N, int K, int M)
{
    (void)N;
    skinny_plan_t p{SKINNY_KIND_LOOP_K, 256, 64, 4, 1, 1, 1, 0, 1, 0};
    if (K % 8 != 0)
        return registry().scalar->plan;
    // Prefer a FIXED_K variant for this K with one row per wave, the
    // non-temporal hint, x in registers, the fewest k_split waves whose x slice
    // fits the register budget, and the widest row groups.
    const Variant *best = nullptr;
    const Registry &reg = registry();
    for (int i = 0; i < reg.n; ++i) {
        const Variant &v = *reg.v[i];
        if (v.plan.kind != SKINNY_KIND_FIXED_K || v.k_fixed != K || v.plan.rows_per_wave != 1 ||
            v.plan.nontemporal != 1 || v.plan.x_in_lds != 0 || v.plan.prefetch != 1 ||
            v.fn[M - 1] == nullptr)
            continue;
        if (!best) {
            best = &v;
            continue;
        }
        if (v.plan.k_split < best->plan.k_split ||
            (v.plan.k_split == best->plan.k_split && v.plan.lanes_per_row > best->plan.lanes_per_row))
            best = &v;
    }
    if (best) {
        p = best->plan;
        p.threads_per_block = 256;
        p.grid_blocks = 0;
    }
    return p;
}

bool lookup_plan(int N, int K, int M, skinny_plan_t *out)
{
    for (int i = 0; i < kNumPlans; ++i) {
        const PlanEntry &e = kPlanTable[i];
        if (e.N == N && e.K == K && e.M == M) {
            *out = e.plan;
            return true;
        }
    }
    *out = default_plan(N, K, M);
    return false;
}

// --- device properties -----------------------------------------------------

constexpr int kMaxDevices = 64;
struct DevInfo {
    int state;        // 0 unknown, 1 gfx950, SKINNY_ERR_* otherwise
    int max_lds;      // bytes of LDS one block may use
    int cus;          // compute units
};
std::mutex g_dev_mu;
DevInfo g_dev[kMaxDevices];

int check_device(int dev, DevInfo *out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return SKINNY_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DevInfo &d = g_dev[dev];
    if (d.state == 0) {
        int count = 0;
        if (hipGetDeviceCount(&count) != hipSuccess || dev >= count) {
            (void)hipGetLastError();
            return SKINNY_ERR_INVALID_ARG;
        }
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return SKINNY_ERR_UNSUPPORTED;
        }
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            d.state = SKINNY_ERR_UNSUPPORTED;
        } else {
            int lds = 0;
            if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
                lds <= 0)
                lds = 65536;
            d.max_lds = lds;
            d.cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
            d.state = 1;
        }
    }
    if (out)
        *out = d;
    return d.state == 1 ? SKINNY_OK : d.state;
}

int current_device(DevInfo *out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return SKINNY_ERR_UNSUPPORTED;
    }
    return check_device(dev, out);
}

// --- validation --------------------------------------------------------------

bool overlaps(const void *a, size_t la, const void *b, size_t lb)
{
    if (!a || !b || la == 0 || lb == 0)
        return false;
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + lb && pb < pa + la;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Call {
    const void *x, *x1;  // x of W0 and of W1 (x1 == x for the shared-input pair)
    const void *w0, *w1;
    void *y0, *y1;
    int M, N, K, nmats;
    int ldx, ldy;        // row strides of x/x1 and y0/y1, in elements
    int out_f32;         // 1: float32 outputs, 0: bfloat16
};

Call single_call(const void *x, const void *W, void *y, int M, int N, int K, int out_f32)
{
    return Call{x, x, W, nullptr, y, nullptr, M, N, K, 1, K, N, out_f32};
}

// Bytes spanned by `rows` rows of `width` elements at `stride` elements.
size_t span(int rows, int width, int stride, size_t elem)
{
    return rows > 0 && width > 0 ? ((size_t)(rows - 1) * stride + width) * elem : 0;
}

// Two same-shape row-strided blocks (rows x width at the same stride, in bytes)
// share no byte. Exact when the strides are equal: the second block's rows must
// fall in the gaps between the first block's rows, or the spans must not meet.
bool strided_disjoint(const void *p, const void *q, int rows, size_t width, size_t stride)
{
    const size_t s = (size_t)(rows - 1) * stride + width;
    if (!overlaps(p, s, q, s))
        return true;
    const long long d = (long long)(reinterpret_cast<uintptr_t>(q) - reinterpret_cast<uintptr_t>(p));
    const long long st = (long long)stride;
    const long long r = ((d % st) + st) % st;  // q's rows start r bytes into p's stride period
    return r >= (long long)width && r + (long long)width <= st;
}

int validate(const Call &c)
{
    if (c.M < 0 || c.M > 4 || c.N < 0 || c.K < 0)
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
bool vector_ok(const Call &c)
{
    const bool al = aligned(c.x, 16) && aligned(c.w0, 16) &&
                    (c.nmats == 1 || (aligned(c.w1, 16) && aligned(c.x1, 16)));
    return al && c.K % 8 == 0 && c.ldx % 8 == 0 && c.K <= (1 << 20) &&
           span(c.M, c.K, c.ldx, 2) < (1u << 31);
}

// The MFMA family needs whole batches of 128 * chunks in every k_split slice.
bool mfma_k_ok(const skinny_plan_t &p, int K)
{
    const int per = 128 * p.k_split;
    return K % per == 0 && (K / per) % p.chunks == 0;
}

int plan_ok(const skinny_plan_t &p, const Variant *v)
{
    if (!v)
        return SKINNY_ERR_UNSUPPORTED;
    const int tpb = p.threads_per_block;
    if (tpb < 64 || tpb > skg::kMaxWaves * 64 || tpb % 64 != 0 || (tpb / 64) % p.k_split != 0)
        return SKINNY_ERR_INVALID_ARG;
    if (p.grid_blocks < 0)
        return SKINNY_ERR_INVALID_ARG;
    if (p.kind == SKINNY_KIND_SCALAR && tpb != 256)
        return SKINNY_ERR_INVALID_ARG;
    if (p.x_in_lds != 0 && p.x_in_lds != 1)
        return SKINNY_ERR_INVALID_ARG;
    if (p.prefetch < 0 || p.prefetch > (p.kind == SKINNY_KIND_FIXED_K ? 2 : 1))
        return SKINNY_ERR_INVALID_ARG;
    return SKINNY_OK;
}

// Launch and, on failure, clear the runtime's sticky last-error so that a refused
// launch is reported once, here, and not again by the caller's next HIP call.
hipError_t launch(const void *fn, int grid, int block, size_t lds, void **args, hipStream_t s)
{
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)block), args, lds, s);
    if (e != hipSuccess)
        (void)hipGetLastError();
    return e;
}

std::atomic<int> g_lds_raised[kNumAll][4];
std::atomic<int> g_static_lds[kNumAll][4];  // static LDS bytes + 1 (0 = not queried)

// Static LDS of a kernel (its __shared__ arrays), queried once.
int static_lds(int vidx, int M, const void *fn)
{
    std::atomic<int> &slot = g_static_lds[vidx][M - 1];
    int v = slot.load(std::memory_order_acquire);
    if (v > 0)
        return v - 1;
    hipFuncAttributes attr{};
    if (hipFuncGetAttributes(&attr, fn) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    slot.store((int)attr.sharedSizeBytes + 1, std::memory_order_release);
    return (int)attr.sharedSizeBytes;
}

// Blocks of this kernel one CU holds at once (cached per kernel, block size
// and LDS size; 1 if the query fails).
struct OccEntry {
    int vidx, M, tpb;
    size_t lds;
    int blocks;
};
std::mutex g_occ_mu;
OccEntry g_occ[512];
int g_occ_n = 0;

int blocks_per_cu(int vidx, int M, const void *fn, int tpb, size_t lds)
{
    std::lock_guard<std::mutex> lk(g_occ_mu);
    for (int i = 0; i < g_occ_n; ++i)
        if (g_occ[i].vidx == vidx && g_occ[i].M == M && g_occ[i].tpb == tpb && g_occ[i].lds == lds)
            return g_occ[i].blocks;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, tpb, lds) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        n = 1;
    }
    if (g_occ_n < (int)(sizeof(g_occ) / sizeof(g_occ[0])))
        g_occ[g_occ_n++] = OccEntry{vidx, M, tpb, lds, n};
    return n;
}

int run(const Call &c, const skinny_plan_t *plan_in, hipStream_t stream)
{
    int st = validate(c);
    if (st != SKINNY_OK)
        return st;
    if (plan_in) {
        const Variant *v = find_variant(*plan_in);
        st = plan_ok(*plan_in, v);
        if (st != SKINNY_OK)
            return st;
        if (v->plan.kind == SKINNY_KIND_FIXED_K && c.K != v->k_fixed && c.K != 0)
            return SKINNY_ERR_INVALID_ARG;
        if (c.M > 0 && v->fn[c.M - 1] == nullptr)
            return SKINNY_ERR_UNSUPPORTED;
        if (c.M > 0 && c.N > 0 && c.K > 0 && v->plan.kind != SKINNY_KIND_SCALAR && !vector_ok(c))
            return SKINNY_ERR_INVALID_ARG;
        if (c.K > 0 && v->plan.kind == SKINNY_KIND_MFMA && !mfma_k_ok(v->plan, c.K))
            return SKINNY_ERR_INVALID_ARG;
    }
    if (c.M == 0 || c.N == 0)
        return SKINNY_OK;

    DevInfo dev{};
    st = current_device(&dev);
    if (st != SKINNY_OK)
        return st;

    if (c.K == 0) {
        long long count = (long long)c.M * c.N;
        void *y0 = c.y0;
        void *y1 = c.nmats == 2 ? c.y1 : nullptr;
        int n = c.N, ldy = c.ldy;
        int elem = c.out_f32 ? 4 : 2;
        void *args[] = {&y0, &y1, &n, &ldy, &count, &elem};
        const long long blocks = (count + 255) / 256;
        if (blocks > 0x7FFFFFFF)
            return SKINNY_ERR_INVALID_ARG;
        return launch(reinterpret_cast<const void *>(&skg::zero_kernel), (int)blocks, 256, 0, args,
                      stream) == hipSuccess
                   ? SKINNY_OK
                   : SKINNY_ERR_LAUNCH;
    }

    skinny_plan_t plan;
    if (plan_in)
        plan = *plan_in;
    else
        lookup_plan(c.N, c.K, c.M, &plan);

    const bool vec = vector_ok(c);
    if (!vec && plan.kind != SKINNY_KIND_SCALAR) {
        if (plan_in)
            return SKINNY_ERR_INVALID_ARG;
        plan = registry().scalar->plan;
    }
    if (!plan_in && plan.kind == SKINNY_KIND_FIXED_K) {
        const Variant *v = find_variant(plan);
        if (!v || v->k_fixed != c.K || !v->fn[c.M - 1])
            plan = default_plan(c.N, c.K, c.M);
    }
    if (!plan_in && plan.kind == SKINNY_KIND_MFMA && !mfma_k_ok(plan, c.K))
        plan = default_plan(c.N, c.K, c.M);
    const Variant *v = find_variant(plan);
    if (!v || plan_ok(plan, v) != SKINNY_OK || !v->fn[c.M - 1])
        return SKINNY_ERR_UNSUPPORTED;

    skg::Args a{};
    a.x = static_cast<const uint16_t *>(c.x);
    a.x1 = static_cast<const uint16_t *>(c.nmats == 2 ? c.x1 : c.x);
    a.w0 = static_cast<const uint16_t *>(c.w0);
    a.w1 = static_cast<const uint16_t *>(c.nmats == 2 ? c.w1 : c.w0);
    a.y0 = c.y0;
    a.y1 = c.nmats == 2 ? c.y1 : c.y0;
    a.N = c.N;
    a.K = c.K;
    a.ldx = c.ldx;
    a.ldy = c.ldy;
    a.nmats = c.nmats;
    a.out_f32 = c.out_f32;

    const int vidx = (int)(v - kAllVariants);
    hipError_t err;
    auto launch_scalar = [&]() {
        const long long blocks = ((long long)c.nmats * c.N + 3) / 4;  // one wave per output row
        a.tiles = 0;
        void *args[] = {&a};
        return launch(registry().scalar->fn[c.M - 1], (int)blocks, 256, 0, args, stream);
    };
    if (plan.kind == SKINNY_KIND_SCALAR) {
        err = launch_scalar();
    } else {
        const int waves = plan.threads_per_block / 64;
        const long long rows_per_tile = (long long)(waves / plan.k_split) * v->rows_per_group;
        const long long tiles = ((long long)c.N + rows_per_tile - 1) / rows_per_tile;
        if (tiles > (1LL << 30))  // keeps the tile indices the kernels compute inside int
            return SKINNY_ERR_INVALID_ARG;
        // every buffer resource spans at most one wave group's rows
        if ((long long)v->rows_per_group * c.K * 2 > 0x7FFFFFFFLL)
            return plan_in ? SKINNY_ERR_INVALID_ARG : SKINNY_ERR_UNSUPPORTED;
        // and one output row (N elements) of y
        if ((long long)c.N * (c.out_f32 ? 4 : 2) > 0x7FFFFFFFLL) {
            if (plan_in)
                return SKINNY_ERR_UNSUPPORTED;
            err = launch_scalar();
            return err == hipSuccess ? SKINNY_OK : SKINNY_ERR_LAUNCH;
        }
        a.tiles = (int)tiles;
        // Dynamic LDS: x staged as [M][Kpad] (LOOP_K) or [M][K] (MFMA).
        int kpad = c.K;
        size_t lds = 0;
        if (plan.kind == SKINNY_KIND_LOOP_K) {
            const int kstep = 512 * plan.chunks;
            kpad = ((c.K + kstep - 1) / kstep) * kstep;
            lds = (size_t)c.M * kpad * 2;
        } else if (plan.kind == SKINNY_KIND_MFMA) {
            lds = (size_t)c.M * c.K * 2;
        }
        const void *fn = v->fn[c.M - 1];
        const int block = plan.threads_per_block;
        const int st_lds = lds > 0 ? static_lds(vidx, c.M, fn) : 0;
        if (st_lds < 0)
            return SKINNY_ERR_LAUNCH;
        if (lds + (size_t)st_lds > (size_t)dev.max_lds) {
            if (plan_in)
                return SKINNY_ERR_UNSUPPORTED;
            err = launch_scalar();  // x does not fit in LDS: element-wise path
            return err == hipSuccess ? SKINNY_OK : SKINNY_ERR_LAUNCH;
        }
        if (lds > 65536 && !g_lds_raised[vidx][c.M - 1].load(std::memory_order_acquire)) {
            // allow this kernel the whole LDS of a block beside its static arrays
            if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    dev.max_lds - st_lds) != hipSuccess) {
                (void)hipGetLastError();
                return SKINNY_ERR_LAUNCH;
            }
            g_lds_raised[vidx][c.M - 1].store(1, std::memory_order_release);
        }
        // Blocks per weight: one per tile, or a persistent grid that fills the device
        // once (grid_blocks == 0), or at most grid_blocks; a pair launches the same
        // count for each weight (even blocks W0, odd blocks W1).
        long long cap = plan.grid_blocks > 0
                            ? plan.grid_blocks
                            : (long long)dev.cus * blocks_per_cu(vidx, c.M, fn, block, lds);
        cap = (cap + c.nmats - 1) / c.nmats;
        if (cap < 1)
            cap = 1;
        const long long per = tiles < cap ? tiles : cap;
        const int grid = (int)(per * c.nmats);
        if (plan.kind == SKINNY_KIND_LOOP_K) {
            void *args[] = {&a, &kpad};
            err = launch(fn, grid, block, lds, args, stream);
        } else {
            void *args[] = {&a};
            err = launch(fn, grid, block, lds, args, stream);
        }
    }
    return err == hipSuccess ? SKINNY_OK : SKINNY_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int skinny_gemm_init(int device) { return check_device(device, nullptr); }

int skinny_gemm_bf16(const void *x, const void *W, void *y, int M, int N, int K, hipStream_t stream)
{
    return run(single_call(x, W, y, M, N, K, 0), nullptr, stream);
}

int skinny_gemm_bf16_pair(const void *x, const void *W0, const void *W1, void *y0, void *y1, int M,
                          int N, int K, hipStream_t stream)
{
    return run(Call{x, x, W0, W1, y0, y1, M, N, K, 2, K, N, 0}, nullptr, stream);
}

int skinny_gemm_bf16_ex(const void *x, const void *W, void *y, int M, int N, int K,
                        const skinny_plan_t *plan, hipStream_t stream)
{
    if (!plan)
        return SKINNY_ERR_INVALID_ARG;
    return run(single_call(x, W, y, M, N, K, 0), plan, stream);
}

int skinny_gemm_bf16_pair_ex(const void *x, const void *W0, const void *W1, void *y0, void *y1,
                             int M, int N, int K, const skinny_plan_t *plan, hipStream_t stream)
{
    if (!plan)
        return SKINNY_ERR_INVALID_ARG;
    return run(Call{x, x, W0, W1, y0, y1, M, N, K, 2, K, N, 0}, plan, stream);
}

int skinny_gemm_bf16_pair_strided(const void *x0, const void *x1, int ldx, const void *W0,
                                  const void *W1, void *y0, void *y1, int ldy, int M, int N, int K,
                                  hipStream_t stream)
{
    return run(Call{x0, x1, W0, W1, y0, y1, M, N, K, 2, ldx, ldy, 0}, nullptr, stream);
}

int skinny_gemm_bf16_pair_strided_ex(const void *x0, const void *x1, int ldx, const void *W0,
                                     const void *W1, void *y0, void *y1, int ldy, int M, int N,
                                     int K, const skinny_plan_t *plan, hipStream_t stream)
{
    if (!plan)
        return SKINNY_ERR_INVALID_ARG;
    return run(Call{x0, x1, W0, W1, y0, y1, M, N, K, 2, ldx, ldy, 0}, plan, stream);
}

int skinny_gemm_bf16_f32out(const void *x, const void *W, float *y, int M, int N, int K,
                            hipStream_t stream)
{
    return run(single_call(x, W, y, M, N, K, 1), nullptr, stream);
}

int skinny_gemm_bf16_f32out_ex(const void *x, const void *W, float *y, int M, int N, int K,
                               const skinny_plan_t *plan, hipStream_t stream)
{
    if (!plan)
        return SKINNY_ERR_INVALID_ARG;
    return run(single_call(x, W, y, M, N, K, 1), plan, stream);
}

int skinny_gemm_get_plan(int N, int K, int M, skinny_plan_t *out)
{
    if (!out || N < 1 || K < 1 || M < 1 || M > 4)
        return SKINNY_ERR_INVALID_ARG;
    return lookup_plan(N, K, M, out) ? 1 : 0;
}

int skinny_gemm_num_variants(void) { return registry().n; }

int skinny_gemm_get_variant(int index, skinny_plan_t *out)
{
    const Registry &r = registry();
    if (!out || index < 0 || index >= r.n)
        return SKINNY_ERR_INVALID_ARG;
    *out = r.v[index]->plan;
    return SKINNY_OK;
}

const char *skinny_gemm_status_string(int status)
{
    switch (status) {
    case SKINNY_OK:
        return "SKINNY_OK: success";
    case SKINNY_ERR_INVALID_ARG:
        return "SKINNY_ERR_INVALID_ARG: invalid argument (pointer, size, overlap or plan)";
    case SKINNY_ERR_UNSUPPORTED:
        return "SKINNY_ERR_UNSUPPORTED: no usable gfx950 device or no compiled variant for this plan";
    case SKINNY_ERR_NOT_INITIALIZED:
        return "SKINNY_ERR_NOT_INITIALIZED: library not initialised";
    case SKINNY_ERR_LAUNCH:
        return "SKINNY_ERR_LAUNCH: the HIP runtime refused the kernel launch";
    default:
        return "SKINNY_ERR_UNKNOWN: unknown status code";
    }
}

int skinny_gemm_version(void) { return kVersion; }

}  // extern "C"
