// Cross-block split-K (include/skinny_gemm.h, skinny_gemm_bf16_split_k): the K
// range of every row is cut into S slices taken by S different blocks, whose
// float32 partial sums meet in a global workspace; the last block of a tile to
// arrive adds them in slice order and writes the output. One launch, no second
// reduce kernel: the single-launch form of the split-K + reduce kernel pair that
// vLLM PR #65306 (SM90 skinny GEMM plans), section Details, counts against
// cuBLAS on its small-N / large-K shapes.
//
// Per slice the arithmetic is that of the compile-time-K kernel (kernels.hpp,
// fixed_k_kernel) with k_split = S: lane (sub, kl) of a wave reads, for row
// r * 64/LPR + sub and chunk j < CH, the 8 elements at s*KS + j*LPR*8 + kl*8 with
// KS = LPR*8*CH; products go through v_dot2c_f32_bf16 in chunk order, the lanes
// of a row meet by the same DPP butterfly, and the S slice sums are added as
// ((p0 + p1) + p2) + ... So a split-K plan gives the same bits as the in-block
// plan with the same (lanes_per_row, chunks, k_split = S).
//
// Hand-off between blocks, with no block ever waiting for another:
//   1. every lane that holds a row sum stores it to part[s][m][row] as an
//      agent-scope atomic store (on gfx950 a store with the sc1 bit: coherent
//      across the eight XCDs' L2 caches by itself);
//   2. each wave waits until its stores are complete (vmcnt 0), then the block
//      meets at a barrier;
//   3. one thread adds 1 to the tile's arrival counter (an agent-scope atomic, so
//      it is issued after every partial of the block is visible device-wide); the
//      block that sees S - 1 there is the last of its tile;
//   4. the last block reads the S partials of each of its outputs with agent-scope
//      atomic loads (sc1: not served by a stale line of its own L2), adds them in
//      slice order, rounds once to bfloat16, stores y, and sets the counter back
//      to 0.
// No fence is used: an agent-scope release or acquire fence writes back or
// invalidates the whole L2 of the XCD, and with one per block the kernel ran
// 10-40x slower than the in-block plans. Counters therefore hold 0 between calls;
// partials are always written before they are read, so they need no clearing.
#include "skinny_gemm.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "kernels.hpp"
#include "validate.hpp"

namespace skg {

struct SplitArgs {
    const uint16_t *x;   // [M][K], contiguous
    const uint16_t *w;   // [N][K]
    uint16_t *y;         // [M][N] bfloat16
    float *part;         // [S][M][N] float32 partial sums
    unsigned *count;     // [tiles] arrival counters, 0 between calls
    int N, K, splits, tiles;
};

// s_waitcnt operand (gfx9 encoding): vmcnt 0, expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

template <int M, int LPR, int CH, int R, bool NT>
__global__ __launch_bounds__(kMaxWaves * 64) void split_k_kernel(SplitArgs a)
{
    constexpr int KS = LPR * 8 * CH;
    constexpr int RPI = 64 / LPR;
    constexpr int ROWS_W = R * RPI;
    constexpr int OUT = sum_lane<LPR>();
    const int rows_t = (int)(blockDim.x >> 6) * ROWS_W;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane / LPR;
    const int kl = lane % LPR;
    // the S blocks of a tile are consecutive, so they run and finish together
    const int tile = __builtin_amdgcn_readfirstlane((int)blockIdx.x / a.splits);
    const int s = __builtin_amdgcn_readfirstlane((int)blockIdx.x - tile * a.splits);
    const int K = a.K;
    const unsigned kbase = (unsigned)(s * KS + kl * 8);

    // this wave's rows: a resource ending at the last valid one (rows >= N read 0)
    const int row0 = tile * rows_t + wave * ROWS_W;
    int valid = a.N - row0;
    valid = valid < 0 ? 0 : (valid > ROWS_W ? ROWS_W : valid);
    const __amdgpu_buffer_rsrc_t ws =
        make_rsrc(valid > 0 ? a.w + (size_t)row0 * K : a.w, (unsigned)(valid * K * 2));
    const __amdgpu_buffer_rsrc_t xs = make_rsrc(a.x, (unsigned)(M * K * 2));

    u32x4 wv[R][CH], xr[M][CH];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < CH; ++j)
            wv[r][j] = load16<NT>(ws, ((unsigned)((r * RPI + sub) * K) + kbase + j * LPR * 8) * 2u);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < CH; ++j)
            xr[m][j] = load16<false>(xs, ((unsigned)(m * K) + kbase + j * LPR * 8) * 2u);

    float acc[M][R];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[m][r] = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[m][r] = dot8(wv[r][j], xr[m][j], acc[m][r]);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[m][r] = group_sum<LPR>(acc[m][r]);

    // 1. partial sums of this slice
    const size_t plane = (size_t)M * a.N;
    if (kl == OUT) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r * RPI + sub;
            if (row < a.N) {
#pragma unroll
                for (int m = 0; m < M; ++m)
                    __hip_atomic_store(&a.part[(size_t)s * plane + (size_t)m * a.N + row], acc[m][r],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    // 2.-3. wait for them, then count this block in
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned before =
            __hip_atomic_fetch_add(&a.count[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = before == (unsigned)(a.splits - 1);
    }
    __syncthreads();
    if (!last)
        return;  // block-uniform

    // 4. the last block of the tile: every slice's partials are complete
    const int base = tile * rows_t;
    for (int i = (int)threadIdx.x; i < M * rows_t; i += (int)blockDim.x) {
        const int m = i / rows_t;
        const int row = base + (i - m * rows_t);
        if (row < a.N) {
            const size_t o = (size_t)m * a.N + row;
            float v = __hip_atomic_load(&a.part[o], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int q = 1; q < a.splits; ++q)
                v += __hip_atomic_load(&a.part[(size_t)q * plane + o], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            a.y[o] = f32_to_bf16(v);
        }
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&a.count[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sets n words to zero (the counters of the library's static workspace).
__global__ void clear_words_kernel(unsigned *p, int n)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n)
        p[i] = 0u;
}

}  // namespace skg

namespace {

using namespace skg_host;

// --- compiled split-K variants ---------------------------------------------

struct SplitVariant {
    skinny_plan_t plan;       // k_split = 0 in the table: S is chosen per call
    const void *fn[kMaxM];    // NULL where x and the weights would not fit the register budget
    int slice_k;              // KS = lanes_per_row * 8 * chunks
    int rows_per_group;       // rows one wave covers
};

// Registers per lane: x takes 4*M*CH VGPRs, the weights 4*R*CH, the sums M*R;
// the same budget as the compile-time-K family with x in registers.
constexpr bool split_fits(int M, int CH, int R) { return M * CH <= 32 && 4 * (M * CH + R * CH) + M * R <= 200; }

template <int M, int LPR, int CH, int R>
constexpr const void *split_fn()
{
    if constexpr (split_fits(M, CH, R))
        return reinterpret_cast<const void *>(&skg::split_k_kernel<M, LPR, CH, R, true>);
    else
        return nullptr;
}

template <int LPR, int CH, int R>
SplitVariant split_variant()
{
    SplitVariant v{};
    v.plan = skinny_plan_t{SKINNY_KIND_SPLIT_K, 256, LPR, CH, R, 0, 1, 0, 0, 0};
    v.fn[0] = split_fn<1, LPR, CH, R>();
    v.fn[1] = split_fn<2, LPR, CH, R>();
    v.fn[2] = split_fn<3, LPR, CH, R>();
    v.fn[3] = split_fn<4, LPR, CH, R>();
    v.fn[4] = split_fn<5, LPR, CH, R>();
    v.fn[5] = split_fn<6, LPR, CH, R>();
    v.fn[6] = split_fn<7, LPR, CH, R>();
    v.fn[7] = split_fn<8, LPR, CH, R>();
    v.slice_k = LPR * 8 * CH;
    v.rows_per_group = R * (64 / LPR);
    return v;
}

// Slices of 512..4096 elements at 64 lanes per row (K = 1024..32768 over 2..8
// slices), and of 256 / 512 / 768 at 32 lanes per row (K = 1536 in two).
const SplitVariant kSplit[] = {
    split_variant<64, 1, 1>(), split_variant<64, 2, 1>(), split_variant<64, 4, 1>(), split_variant<64, 8, 1>(),
    split_variant<64, 1, 2>(), split_variant<64, 2, 2>(), split_variant<64, 4, 2>(),
    split_variant<32, 1, 1>(), split_variant<32, 2, 1>(), split_variant<32, 3, 1>(),
};
constexpr int kNumSplit = sizeof(kSplit) / sizeof(kSplit[0]);

const SplitVariant *find_split(const skinny_plan_t &p)
{
    for (const SplitVariant &v : kSplit)
        if (v.plan.lanes_per_row == p.lanes_per_row && v.plan.chunks == p.chunks &&
            v.plan.rows_per_wave == p.rows_per_wave)
            return &v;
    return nullptr;
}

// Default split-K plan for K: 256 threads, one row per wave, 64 lanes per row
// before 32, and the first slice count of 4, 2, 8 whose slice K / S a compiled
// variant covers (K = 4096: 4 slices of 1024; K = 1536: 2 of 768 at 32 lanes).
bool default_split(int K, int M, skinny_plan_t *out)
{
    const int order[] = {4, 2, 8};
    for (int lpr : {64, 32}) {
        for (int S : order) {
            if (K % S != 0)
                continue;
            for (const SplitVariant &v : kSplit) {
                if (v.plan.lanes_per_row == lpr && v.plan.rows_per_wave == 1 && v.slice_k * S == K &&
                    v.fn[M - 1]) {
                    *out = v.plan;
                    out->k_split = S;
                    return true;
                }
            }
        }
    }
    return false;
}

static_assert(kSplitMaxThreads == skg::kMaxWaves * 64, "split-K block limit");

int split_plan_ok(const skinny_plan_t &p, const SplitVariant *v, int K, int M)
{
    if (p.kind != SKINNY_KIND_SPLIT_K)
        return SKINNY_ERR_INVALID_ARG;
    if (!v)
        return SKINNY_ERR_UNSUPPORTED;
    if (!split_fields_ok(p) || K != v->slice_k * p.k_split)
        return SKINNY_ERR_INVALID_ARG;
    if (!v->fn[M - 1])
        return SKINNY_ERR_UNSUPPORTED;
    return SKINNY_OK;
}

SplitLayout layout_of(const skinny_plan_t &p, const SplitVariant *v, int M, int N)
{
    return split_layout(p.threads_per_block, v->rows_per_group, p.k_split, M, N);
}

// A resolved split-K call: plan, variant and layout, all checked.
struct SplitCall {
    skinny_plan_t plan;
    const SplitVariant *v;
    SplitLayout lay;
};

// Checks of a split-K call that need no device: the common argument checks, the
// vector-path conditions and the plan. *empty is set for calls with nothing to do.
int split_prepare(const Call &c, const skinny_plan_t *plan_in, SplitCall *out, bool *empty)
{
    *empty = false;
    int st = validate(c);
    if (st != SKINNY_OK)
        return st;
    if (c.M == 0 || c.N == 0) {
        *empty = true;
        return SKINNY_OK;
    }
    if (!split_call_ok(c))
        return SKINNY_ERR_INVALID_ARG;
    skinny_plan_t p;
    if (plan_in) {
        p = *plan_in;
    } else if (!default_split(c.K, c.M, &p)) {
        return SKINNY_ERR_UNSUPPORTED;
    }
    const SplitVariant *v = find_split(p);
    st = split_plan_ok(p, v, c.K, c.M);
    if (st != SKINNY_OK)
        return st;
    // each wave's buffer resource spans its rows; partial and output indices fit
    if ((long long)v->rows_per_group * c.K * 2 > 0x7FFFFFFFLL)
        return SKINNY_ERR_INVALID_ARG;
    out->plan = p;
    out->v = v;
    out->lay = layout_of(p, v, c.M, c.N);
    if (!split_layout_ok(out->lay, p.k_split))
        return SKINNY_ERR_INVALID_ARG;
    return SKINNY_OK;
}

hipError_t split_launch(const Call &c, const SplitCall &sc, void *workspace, hipStream_t stream)
{
    skg::SplitArgs a{};
    a.x = static_cast<const uint16_t *>(c.x);
    a.w = static_cast<const uint16_t *>(c.w0);
    a.y = static_cast<uint16_t *>(c.y0);
    a.count = static_cast<unsigned *>(workspace);
    a.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + kSplitPartOffset);
    a.N = c.N;
    a.K = c.K;
    a.splits = sc.plan.k_split;
    a.tiles = (int)sc.lay.tiles;
    void *args[] = {&a};
    const long long grid = (long long)sc.lay.tiles * sc.plan.k_split;
    const hipError_t e = hipLaunchKernel(sc.v->fn[c.M - 1], dim3((unsigned)grid),
                                         dim3((unsigned)sc.plan.threads_per_block), args, 0, stream);
    if (e != hipSuccess)
        (void)hipGetLastError();
    return e;
}

int check_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return SKINNY_ERR_UNSUPPORTED;
    }
    return skinny_gemm_init(dev);
}

// --- the library's own workspace, for callers that cannot allocate -----------

// Largest partials skinny_gemm_bf16_split_k_noalloc serves: 4 MiB (S*M*N <= 2^20).
constexpr size_t kScratchPartBytes = (size_t)4 << 20;
constexpr size_t kScratchBytes = kSplitPartOffset + kScratchPartBytes;

}  // namespace

// One copy per GPU, in the workspace layout above, held from the library's load
// until the process ends. In host code this name is only a handle for
// hipGetSymbolAddress: each GPU's copy has its own device address, which that
// call returns and which is all the kernels are ever given (g_scratch_ptr).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
// per device: 0 nothing done, 2 address known (counters not yet cleared), 1 ready
std::atomic<int> g_scratch_state[64];
void *g_scratch_ptr[64];

// Looks up the current device's copy of `scratch` (caller holds g_scratch_mu).
int scratch_lookup_locked(int dev)
{
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return SKINNY_ERR_LAUNCH;  // nothing recorded: a later call tries again
    }
    g_scratch_ptr[dev] = p;
    g_scratch_state[dev].store(2, std::memory_order_release);
    return SKINNY_OK;
}

// Device address of the current GPU's copy of `scratch`, ready for a call on
// `stream`. The address is looked up once per device, with that device current
// (by skinny_gemm_init, or else here); the first call on the device also enqueues,
// on its stream, a kernel that zeroes the copy's counters (static storage starts at
// zero; the kernel makes it explicit, and a captured first call records it in its
// graph). Later calls find the counters at zero, as every call leaves them.
int scratch_ptr(hipStream_t stream, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return SKINNY_ERR_UNSUPPORTED;
    }
    if (dev < 0 || dev >= 64)
        return SKINNY_ERR_UNSUPPORTED;
    if (g_scratch_state[dev].load(std::memory_order_acquire) != 1) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        int state = g_scratch_state[dev].load(std::memory_order_relaxed);
        if (state == 0) {
            const int st = scratch_lookup_locked(dev);
            if (st != SKINNY_OK)
                return st;
            state = 2;
        }
        if (state == 2) {
            unsigned *cnt = static_cast<unsigned *>(g_scratch_ptr[dev]);
            int n = (int)kSplitCountWords;
            void *args[] = {&cnt, &n};
            if (hipLaunchKernel(reinterpret_cast<const void *>(&skg::clear_words_kernel),
                                dim3((unsigned)((n + 255) / 256)), dim3(256), args, 0, stream) != hipSuccess) {
                (void)hipGetLastError();
                return SKINNY_ERR_LAUNCH;  // still 2: the next call clears them
            }
            g_scratch_state[dev].store(1, std::memory_order_release);
        }
    }
    *out = g_scratch_ptr[dev];
    return SKINNY_OK;
}

}  // namespace

namespace skg_host {

int split_k_scratch_setup(int dev)
{
    if (dev < 0 || dev >= 64)
        return SKINNY_ERR_UNSUPPORTED;
    if (g_scratch_state[dev].load(std::memory_order_acquire) != 0)
        return SKINNY_OK;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_state[dev].load(std::memory_order_relaxed) != 0)
        return SKINNY_OK;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) {
        (void)hipGetLastError();
        return SKINNY_ERR_UNSUPPORTED;
    }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) {
        (void)hipGetLastError();
        return SKINNY_ERR_UNSUPPORTED;
    }
    const int st = scratch_lookup_locked(dev);
    if (prev != dev && hipSetDevice(prev) != hipSuccess)
        (void)hipGetLastError();
    return st;
}

}  // namespace skg_host

extern "C" {

size_t skinny_gemm_split_k_workspace_bytes(int M, int N, int K, const skinny_plan_t *plan)
{
    if (M < 1 || M > kMaxM || N < 1 || K < 1)
        return 0;
    skinny_plan_t p;
    if (plan) {
        p = *plan;
    } else if (!default_split(K, M, &p)) {
        return 0;
    }
    const SplitVariant *v = find_split(p);
    if (split_plan_ok(p, v, K, M) != SKINNY_OK)
        return 0;
    const SplitLayout l = layout_of(p, v, M, N);
    return split_layout_ok(l, p.k_split) ? l.total : 0;
}

int skinny_gemm_bf16_split_k(const void *x, const void *W, void *y, int M, int N, int K,
                             const skinny_plan_t *plan, void *workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    const Call c = single_call(x, W, y, M, N, K, 0);
    SplitCall sc;
    bool empty = false;
    int st = split_prepare(c, plan, &sc, &empty);
    if (st != SKINNY_OK || empty)
        return st;
    if (!split_workspace_ok(c, workspace, workspace_bytes, sc.lay))
        return SKINNY_ERR_INVALID_ARG;
    st = check_current_device();
    if (st != SKINNY_OK)
        return st;
    return split_launch(c, sc, workspace, stream) == hipSuccess ? SKINNY_OK : SKINNY_ERR_LAUNCH;
}

int skinny_gemm_bf16_split_k_noalloc(const void *x, const void *W, void *y, int M, int N, int K,
                                     const skinny_plan_t *plan, hipStream_t stream)
{
    const Call c = single_call(x, W, y, M, N, K, 0);
    SplitCall sc;
    bool empty = false;
    int st = split_prepare(c, plan, &sc, &empty);
    if (st != SKINNY_OK || empty)
        return st;
    if (sc.lay.part_bytes > kScratchPartBytes)
        return SKINNY_ERR_INVALID_ARG;
    st = check_current_device();
    if (st != SKINNY_OK)
        return st;
    void *ws = nullptr;
    st = scratch_ptr(stream, &ws);
    if (st != SKINNY_OK)
        return st;
    return split_launch(c, sc, ws, stream) == hipSuccess ? SKINNY_OK : SKINNY_ERR_LAUNCH;
}

int skinny_gemm_split_k_num_variants(void) { return kNumSplit; }

int skinny_gemm_split_k_get_variant(int index, skinny_plan_t *out)
{
    if (index < 0 || index >= kNumSplit || !out)
        return SKINNY_ERR_INVALID_ARG;
    *out = kSplit[index].plan;
    return SKINNY_OK;
}

int skinny_gemm_split_k_default_plan(int M, int N, int K, skinny_plan_t *out)
{
    if (!out || M < 1 || M > kMaxM || N < 1 || K < 1)
        return SKINNY_ERR_INVALID_ARG;
    return default_split(K, M, out) ? SKINNY_OK : SKINNY_ERR_UNSUPPORTED;
}

}  // extern "C"
