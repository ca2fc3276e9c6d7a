// Device code of the BF16 skinny GEMM for gfx950 (CDNA4, wave64).
//
// y[m, n] = bf16_rne( sum_k x[m, k] * W[n, k] ),  M <= 8 rows of x, W [N][K] row-major
// (or the float32 sum itself, for the float32-output form).
//
// At M <= 8 the product does M flops per weight byte, so its speed is the speed
// at which W streams out of HBM; vLLM PR #65306 (SM90 skinny GEMM plans), section
// Validation, rates such kernels by weight bytes per second against the HBM
// peak. Everything below is arranged around keeping enough 128-bit weight loads
// in flight on every CU:
//
//  * a wavefront reads W with raw buffer loads of 16 bytes per lane; the
//    64 lanes are split into groups of LPR lanes, each group covering one row,
//    so one load instruction touches 64/LPR rows with LPR*16 contiguous bytes
//    each. A buffer resource whose size ends at the last valid row turns the
//    loads of rows >= N into zeros, so the N tail needs no branches;
//  * x (at most 8 rows) stays on chip: in registers (each lane keeps only the K
//    positions it multiplies) or in LDS for the compile-time-K family, in LDS
//    for the looped-K and matrix-core families;
//  * products are accumulated in float32 with v_dot2c_f32_bf16 (two bf16
//    products added into a float32 accumulator per instruction), or on the
//    matrix cores with v_mfma_f32_4x4x4_16b_bf16 (M <= 4);
//  * partial sums of a row meet across its LPR lanes by DPP lane permutations
//    and row broadcasts, then across the k_split waves of a block in LDS,
//    always in one fixed order (deterministic results);
//  * the float32 sum is rounded once to bfloat16, nearest-even, and the M x R
//    results of a lane group are stored together, one store instruction per 16
//    of them, through a buffer resource over the output (rows >= N never stored).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace skg {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Third dword of a gfx9-family buffer resource: 32-bit raw data format, no
// swizzle, so buffer_load_dwordx4 reads 16 plain bytes and reads outside
// [0, num_records) return zero.
constexpr int kBufferFlags = 0x00020000;
// Cache-policy bits of a gfx94x/gfx950 buffer instruction: bit 1 = nt.
constexpr int kAuxNontemporal = 2;
// A byte offset that is always outside the resource: its load returns zeros.
constexpr unsigned kOutOfRange = 0x80000000u;

// Every caller passes a wave-uniform base and size (derived from the block's
// schedule, the tile and the wave index). A buffer resource must sit in scalar
// registers; when the compiler cannot prove an operand uniform (a row clamp that
// it lowers to a vector med3 is enough) it wraps every load that uses the
// resource in a readfirstlane loop, a dozen extra instructions per 16-byte load.
// Taking lane 0's copy of each word here makes the resource scalar once.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes)
{
    const unsigned long long p = (unsigned long long)base;
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)p);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(p >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    void *ub = (void *)(((unsigned long long)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, n, kBufferFlags);
}

template <bool NT>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, unsigned byte_offset)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_offset, 0, NT ? kAuxNontemporal : 0);
}

// Staging of x into LDS, split so that it overlaps the first weight loads:
// stage_issue() loads the first kStageBatch 16-byte pieces per thread (call it
// before issuing weights), stage_finish() writes them to LDS once they arrive
// and copies any rest. Only the waits for these x loads stand between the
// kernel start and the barrier, not one round trip per loop iteration.
// `src(i)` gives the byte offset of piece i in x, or kOutOfRange for zeros.
constexpr int kStageBatch = 8;

template <typename Src>
__device__ __forceinline__ void stage_issue(__amdgpu_buffer_rsrc_t xs, int npieces, Src src,
                                            u32x4 (&t)[kStageBatch])
{
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
        const int i = (int)threadIdx.x + u * (int)blockDim.x;
        t[u] = load16<false>(xs, i < npieces ? src(i) : kOutOfRange);
    }
}

template <typename Src>
__device__ __forceinline__ void stage_finish(__amdgpu_buffer_rsrc_t xs, int npieces, Src src,
                                             const u32x4 (&t)[kStageBatch], u32x4 *dst)
{
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
        const int i = (int)threadIdx.x + u * (int)blockDim.x;
        if (i < npieces)
            dst[i] = t[u];
    }
    for (int i = (int)threadIdx.x + kStageBatch * (int)blockDim.x; i < npieces; i += (int)blockDim.x)
        dst[i] = load16<false>(xs, src(i));
    __syncthreads();
}

// acc + w.lo*x.lo + w.hi*x.hi, the two bfloat16 products exact, float32 sum.
__device__ __forceinline__ float dot2(unsigned w, unsigned x, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, x), acc, false);
}

__device__ __forceinline__ float dot8(const u32x4 &w, const u32x4 &x, float acc)
{
    acc = dot2(w[0], x[0], acc);
    acc = dot2(w[1], x[1], acc);
    acc = dot2(w[2], x[2], acc);
    acc = dot2(w[3], x[3], acc);
    return acc;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __builtin_bit_cast(float, (unsigned)h << 16);
}

// float32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    const unsigned u = __builtin_bit_cast(unsigned, f);
    const unsigned r = u + 0x7FFFu + ((u >> 16) & 1u);
    uint16_t out = (uint16_t)(r >> 16);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        out = (uint16_t)((u >> 16) | 0x0040u);
    return out;
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_add(float v)
{
    // Rows outside ROW_MASK take `old` = 0 and so keep v.
    const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false);
    return v + __builtin_bit_cast(float, moved);
}

// Lane of an LPR-lane group that holds the group's sum after group_sum<LPR>.
template <int LPR>
constexpr int sum_lane() { return LPR >= 32 ? LPR - 1 : 0; }

// Sum over groups of LPR consecutive lanes (LPR = 1, 2, 4, ..., 64). For
// LPR <= 16 every lane of a group ends with the group's sum; for 32 and 64 the
// last lane of the group does (sum_lane). Must run with all 64 lanes active.
// The cross-row steps use the DPP row broadcasts, not the gfx950 permlane
// swaps: clang folds the two results of permlane{16,32}_swap(v, v) into one,
// which silently breaks a butterfly built on them.
template <int LPR>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr (LPR >= 2)
        v = dpp_add<0xB1>(v);        // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (LPR >= 4)
        v = dpp_add<0x4E>(v);        // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LPR >= 8)
        v = dpp_add<0x141>(v);       // row_half_mirror: the other quad of each 8 lanes
    if constexpr (LPR >= 16)
        v = dpp_add<0x140>(v);       // row_mirror: the other half of each 16-lane row
    if constexpr (LPR >= 32)
        v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3: lanes 31, 63 hold 32-sums
    if constexpr (LPR >= 64)
        v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: lane 63 holds the 64-sum
    return v;
}

struct Args {
    const uint16_t *x;   // x of the first (or only) weight: row m at x + m * ldx
    const uint16_t *x1;  // x of the second weight of a pair (== x when it is shared)
    const uint16_t *w0;
    const uint16_t *w1;  // second weight of the pair (== w0 when nmats == 1)
    void *y0;            // bfloat16 or float32 outputs, see out_f32; row m at y + m * ldy
    void *y1;
    int N;
    int K;
    int ldx;             // row stride of x and x1, in elements (>= K)
    int ldy;             // row stride of y0 and y1, in elements (>= N)
    int nmats;           // 1, or 2 for the paired form
    int tiles;           // tiles per weight: ceil(N / rows per tile)
    int out_f32;         // 1: y is float32 (the sum, rounded once to float32); 0: bfloat16
};

// Which weight a block serves and which of its tiles: tile(it) for it = first,
// first + step, ... while tile(it) < a.tiles. For a pair, even blocks serve W0 and
// odd blocks W1 (the host launches an even grid), so a block stages one x only.
struct Sched {
    int mat, first, step;

    __device__ __forceinline__ int tile(int it) const { return it; }
};

__device__ __forceinline__ Sched block_sched(const Args &a)
{
    if (a.nmats == 2)
        return Sched{(int)(blockIdx.x & 1), (int)(blockIdx.x >> 1), (int)(gridDim.x >> 1)};
    return Sched{0, (int)blockIdx.x, (int)gridDim.x};
}

// Bytes of x a block may read: M rows of K elements at stride ldx.
__device__ __forceinline__ unsigned x_bytes(const Args &a, int M)
{
    return (unsigned)(((M - 1) * a.ldx + a.K) * 2);
}

// Store one output element: bfloat16 (nearest-even) or float32, by a block-uniform flag.
__device__ __forceinline__ void store_out(const Args &a, void *ym, size_t idx, float v)
{
    if (a.out_f32)
        static_cast<float *>(ym)[idx] = v;
    else
        static_cast<uint16_t *>(ym)[idx] = f32_to_bf16(v);
}

// f(std::integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// In every 16-lane row, lane 15's v moved to lane 15 - S (DPP row_shl:S).
template <int S>
__device__ __forceinline__ float from_row_end(float v)
{
    if constexpr (S == 0)
        return v;
    else
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x100 + S,
                                                                      0xF, 0xF, false));
}

// All M output rows of ym as one buffer resource: element (m, n) at m * ldy + n.
// The host launches the fast kernels only when that span fits in 31 bits.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const Args &a, void *ym, int M)
{
    const unsigned eb = a.out_f32 ? 4u : 2u;
    return make_rsrc(ym, (unsigned)((M - 1) * a.ldy + a.N) * eb);
}

// Store the M x R results of a lane group: result k = r * M + m (row m of y,
// output row row(r)) goes to the lane whose `slot` is k mod SLOTS, and each
// SLOTS results take one store instruction, issued by every lane with no
// branch: a lane without a result, or whose row is >= N, passes an offset the
// hardware drops. val(k, s) is result k as seen from the lane of slot s (after
// any lane move that takes). One instruction where the rows used to take M x R
// measured 0.2-0.4 us less per call at M = 4 on the decode shapes.
template <int M, int R, int SLOTS, typename Val, typename Row>
__device__ __forceinline__ void store_results(const Args &a, __amdgpu_buffer_rsrc_t yr, int slot, Val &&val,
                                              Row &&row)
{
    constexpr int NV = M * R;
    static_for<0, (NV + SLOTS - 1) / SLOTS>([&](auto bc) {
        constexpr int B = decltype(bc)::value;
        constexpr int NS = NV - B * SLOTS < SLOTS ? NV - B * SLOTS : SLOTS;
        float v = 0.0f;
        static_for<0, NS>([&](auto sc) {
            constexpr int S = decltype(sc)::value;
            const float u = val(std::integral_constant<int, B * SLOTS + S>{}, sc);
            v = slot == S ? u : v;
        });
        const bool has = slot >= 0 && slot < NS;
        const int k = has ? B * SLOTS + slot : 0;
        const int m = k % M;
        const int rw = row(k / M);
        const bool mine = has && rw < a.N;
        const unsigned idx = (unsigned)(m * a.ldy + rw);
        if (a.out_f32)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), yr,
                                                  (int)(mine ? idx * 4u : kOutOfRange), 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), yr, (int)(mine ? idx * 2u : kOutOfRange), 0, 0);
    });
}

// ---------------------------------------------------------------------------
// Family FIXED_K: K = KW * LPR * 8 * CH known at compile time.
//
// A block has W waves (a launch-time value, W % KW == 0) in W/KW groups; the
// KW waves of a group share the same rows and split K into KW slices. A tile
// is the rows the block covers per iteration, (W/KW) * ROWS_W consecutive
// rows; each group owns ROWS_W = R * 64/LPR of them. Lane (sub, kl) =
// (lane / LPR, lane % LPR) reads, for row r*RPI + sub of its group and chunk
// j < CH, the 8 elements starting at  kw * K/KW + j * LPR*8 + kl * 8.
//
// x lives in registers (XL = 0: each lane keeps the M*CH 16-byte pieces it
// multiplies) or in LDS (XL = 1 or 2: the block stages x[M][K] once and every
// chunk reads its pieces back, which frees VGPRs at M >= 3; with XL = 2 the
// pieces of a chunk are read one chunk ahead of their use).
//
// Each block loops over the tiles of one weight (block_sched). PF selects how
// the loop overlaps loads with arithmetic:
//   0  each tile is loaded and then consumed (one register set; suits grids of
//      one tile per block);
//   1  two register sets alternate: the next tile's loads are issued before the
//      current tile is consumed;
//   2  rolling: one register set, and chunk j of the block's next tile is loaded
//      into the registers of chunk j as soon as they have been multiplied, so a
//      wave keeps R*CH loads in flight through the multiply and the reduction
//      however long those take (they grow with M).
// A load for a tile past the last one uses an empty buffer resource and moves
// no data.
// ---------------------------------------------------------------------------
constexpr int kMaxWaves = 8;  // largest block: 512 threads

template <int M, int LPR, int CH, int R, int KW, int XL, bool NT, int PF>
struct FixedK {
    static constexpr int K = KW * LPR * 8 * CH;
    static constexpr int KSLICE = K / KW;
    static constexpr int RPI = 64 / LPR;
    static constexpr int ROWS_W = R * RPI;
    static_assert(64 % LPR == 0 && LPR >= 8, "lanes per row: 8, 16, 32 or 64");
    static_assert(kMaxWaves % KW == 0, "k_split must divide the largest block");

    // Buffer resource over this wave group's rows of tile t of weight wm; a tile
    // past the last one gets an empty resource, whose loads read zeros.
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const Args &a, const uint16_t *wm,
                                                                     int t, int rows_t, int grp)
    {
        const uint16_t *base = wm;
        int valid = 0;
        if (t < a.tiles) {
            const int row0 = t * rows_t + grp * ROWS_W;
            valid = a.N - row0;
            valid = valid < 0 ? 0 : (valid > ROWS_W ? ROWS_W : valid);
            base = wm + (size_t)row0 * K;
        }
        return make_rsrc(base, (unsigned)(valid * K * 2));
    }

    // Byte offset of this lane's chunk j of row r within the group's rows.
    static __device__ __forceinline__ unsigned chunk_off(int r, int sub, unsigned kbase, int j)
    {
        return ((unsigned)((r * RPI + sub) * K) + kbase + j * LPR * 8) * 2u;
    }

    // Issue all weight loads of tile t for this wave's rows.
    static __device__ __forceinline__ void issue(const Args &a, const uint16_t *wm, int t, int rows_t,
                                                 int grp, int sub, unsigned kbase, u32x4 (&wv)[R][CH])
    {
        const __amdgpu_buffer_rsrc_t ws = tile_rsrc(a, wm, t, rows_t, grp);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < CH; ++j)
                wv[r][j] = load16<NT>(ws, chunk_off(r, sub, kbase, j));
    }
};

template <int M, int LPR, int CH, int R, int KW, int XL, bool NT, int PF>
__global__ __launch_bounds__(kMaxWaves * 64) void fixed_k_kernel(Args a)
{
    using F = FixedK<M, LPR, CH, R, KW, XL, NT, PF>;
    constexpr int K = F::K;
    constexpr int KSLICE = F::KSLICE;
    constexpr int RPI = F::RPI;
    constexpr int ROWS_W = F::ROWS_W;
    constexpr int OUT = sum_lane<LPR>();

    // The host launches blockDim.x = 64 * waves with waves % KW == 0.
    const int groups = (int)(blockDim.x >> 6) / KW;
    const int rows_t = groups * ROWS_W;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kw = wave % KW;
    const int grp = wave / KW;
    const int sub = lane / LPR;
    const int kl = lane % LPR;
    const unsigned kbase = (unsigned)(kw * KSLICE + kl * 8);
    const Sched sc = block_sched(a);
    const int step = sc.step;
    const uint16_t *wm = sc.mat ? a.w1 : a.w0;
    const uint16_t *xm = sc.mat ? a.x1 : a.x;
    void *ym = sc.mat ? a.y1 : a.y0;
    const __amdgpu_buffer_rsrc_t yr = out_rsrc(a, ym, M);

    int it = sc.first;
    int tile = sc.tile(it);
    if (tile >= a.tiles)
        return;  // whole block

    __shared__ u32x4 x_lds[XL ? M * K / 8 : 1];
    __shared__ float part[KW > 1 ? kMaxWaves * M * ROWS_W : 1];
    u32x4 wa[R][CH], wb[PF == 1 ? R : 1][PF == 1 ? CH : 1];
    u32x4 xr[XL ? 1 : M][XL ? 1 : CH];
    const __amdgpu_buffer_rsrc_t xs = make_rsrc(xm, x_bytes(a, M));
    const int ldx = a.ldx;
    if constexpr (XL) {
        // x pieces first (L2), then the weights (HBM), then x into LDS as [M][K]
        auto src = [=](int i) {
            const int m = i / (K / 8);
            return (unsigned)(m * ldx + (i - m * (K / 8)) * 8) * 2u;
        };
        u32x4 xt[kStageBatch];
        stage_issue(xs, M * K / 8, src, xt);
        F::issue(a, wm, tile, rows_t, grp, sub, kbase, wa);
        stage_finish(xs, M * K / 8, src, xt, x_lds);
    } else {
        F::issue(a, wm, tile, rows_t, grp, sub, kbase, wa);  // weights first: they come from HBM
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int j = 0; j < CH; ++j)
                xr[m][j] = load16<false>(xs, (unsigned)(m * ldx + (int)kbase + j * LPR * 8) * 2u);
    }

    // With x in LDS, chunk 0's pieces stay in registers for every tile (x is the
    // same for all of them): re-read at each tile start, they waited behind the
    // tile's first weights.
    u32x4 x0[XL ? M : 1];
    if constexpr (XL) {
        const volatile __attribute__((address_space(3))) u32x4 *xp0 =
            (const volatile __attribute__((address_space(3))) u32x4 *)x_lds;
#pragma unroll
        for (int m = 0; m < M; ++m)
            x0[m] = xp0[(m * K + (int)kbase) / 8];
    }

    // Multiply tile t's weights wv, reduce and store; after_chunk(j) runs once
    // chunk j of wv is no longer needed.
    auto consume = [&](int t, const u32x4 (&wv)[R][CH], auto &&after_chunk) {
        float acc[M][R];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[m][r] = 0.0f;
        // x from LDS: XL = 1 reads chunk j's pieces at chunk j; XL = 2 reads them
        // one chunk ahead (before chunk j-1 is multiplied), so the LDS latency
        // hides behind those products, at the price of M more 16-byte registers.
        // volatile: keep each LDS read in its chunk; hoisting them out of the
        // tile loop would rebuild the register copy of x that XL avoids.
        const volatile __attribute__((address_space(3))) u32x4 *xp =
            (const volatile __attribute__((address_space(3))) u32x4 *)x_lds;
        u32x4 xc[XL == 2 ? M : 1], xn[XL == 2 ? M : 1];
        auto read_x = [&](int j, u32x4 (&dst)[XL == 2 ? M : 1]) {
#pragma unroll
            for (int m = 0; m < (XL == 2 ? M : 1); ++m)
                dst[m] = xp[(m * K + (int)kbase + j * LPR * 8) / 8];
        };
        if constexpr (XL == 2) {
#pragma unroll
            for (int m = 0; m < M; ++m)
                xc[m] = x0[m];
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if constexpr (XL == 2) {
                if (j + 1 < CH) {
                    read_x(j + 1, xn);
                    // keep these reads ahead of chunk j's products: left alone, the
                    // scheduler sinks them below most of the chunk, and chunk j+1 then
                    // starts by waiting out the LDS latency
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                u32x4 xv;
                if constexpr (XL == 2)
                    xv = xc[m];
                else if constexpr (XL == 1)
                    xv = j == 0 ? x0[m] : xp[(m * K + (int)kbase + j * LPR * 8) / 8];
                else
                    xv = xr[m][j];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    acc[m][r] = dot8(wv[r][j], xv, acc[m][r]);
                if (m == M - 1)
                    after_chunk(j);
            }
            if constexpr (XL == 2) {
#pragma unroll
                for (int m = 0; m < M; ++m)
                    xc[m] = xn[m];
            }
        }
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[m][r] = group_sum<LPR>(acc[m][r]);

        const int row0 = t * rows_t + grp * ROWS_W;
        auto row = [&](int r) { return row0 + r * RPI + sub; };
        if constexpr (KW == 1) {
            if constexpr (LPR >= 32) {
                // the group's sums sit in its last lane, lane 15 of a 16-lane row
                store_results<M, R, 16>(a, yr, OUT - kl, [&](auto k, auto s) {
                    return from_row_end<decltype(s)::value>(acc[k % M][k / M]);
                }, row);
            } else {
                // every lane of the group holds every sum
                store_results<M, R, LPR>(a, yr, kl, [&](auto k, auto) { return acc[k % M][k / M]; }, row);
            }
        } else {
            if (kl == OUT) {
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        part[((grp * KW + kw) * M + m) * ROWS_W + r * RPI + sub] = acc[m][r];
            }
            __syncthreads();
            // the group's first wave sums and stores (a wave-uniform branch: the
            // other waves issue no stores, so nothing delays their loads)
            if (kw == 0) {
                // every lane of the group reads every sum, one at a time as the
                // stores take them (a table of all M x R would cost registers)
                store_results<M, R, (LPR < 16 ? LPR : 16)>(a, yr, kl, [&](auto k, auto) {
                    constexpr int m = decltype(k)::value % M, r = decltype(k)::value / M;
                    float s = part[((grp * KW + 0) * M + m) * ROWS_W + r * RPI + sub];
#pragma unroll
                    for (int q = 1; q < KW; ++q)
                        s += part[((grp * KW + q) * M + m) * ROWS_W + r * RPI + sub];
                    return s;
                }, row);
            }
            __syncthreads();
        }
    };

    // The block's last tile is consumed outside the prefetch loops, so that no
    // loads are issued for a tile past the end.
    auto nothing = [](int) {};
    if constexpr (PF == 2) {
        while (true) {
            const int next = sc.tile(it + step);
            if (next >= a.tiles)
                break;
            const __amdgpu_buffer_rsrc_t wn = F::tile_rsrc(a, wm, next, rows_t, grp);
            consume(tile, wa, [&](int j) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    wa[r][j] = load16<NT>(wn, F::chunk_off(r, sub, kbase, j));
                // keep these loads between chunk j's products and chunk j+1's: left
                // alone, the scheduler sinks all of them below the last chunk
                __builtin_amdgcn_sched_barrier(0);
            });
            it += step;
            tile = next;
        }
        consume(tile, wa, nothing);
    } else if constexpr (PF == 1) {
        while (true) {
            int next = sc.tile(it + step);
            if (next >= a.tiles) {
                consume(tile, wa, nothing);
                break;
            }
            F::issue(a, wm, next, rows_t, grp, sub, kbase, wb);
            consume(tile, wa, nothing);
            it += step;
            tile = next;
            next = sc.tile(it + step);
            if (next >= a.tiles) {
                consume(tile, wb, nothing);
                break;
            }
            F::issue(a, wm, next, rows_t, grp, sub, kbase, wa);
            consume(tile, wb, nothing);
            it += step;
            tile = next;
        }
    } else {
        while (true) {
            consume(tile, wa, nothing);
            it += step;
            tile = sc.tile(it);
            if (tile >= a.tiles)
                break;
            F::issue(a, wm, tile, rows_t, grp, sub, kbase, wa);
        }
    }
}

// ---------------------------------------------------------------------------
// Family LOOP_K: any K with K % 8 == 0. One wave = one group of R rows (64
// lanes per row); x is staged once per block into LDS as [M][Kpad] with a zero
// tail up to a multiple of 512*U, and the K loop keeps U loads per row in
// flight. Weight chunks past K use an out-of-range offset and read as zeros.
// ---------------------------------------------------------------------------
template <int M, int U, int R, bool NT>
__global__ __launch_bounds__(kMaxWaves * 64) void loop_k_kernel(Args a, int kpad)
{
    extern __shared__ u32x4 lds_x[];  // [M][kpad / 8]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = a.K;
    const int kvec = kpad / 8;
    const Sched sc = block_sched(a);
    if (sc.tile(sc.first) >= a.tiles)
        return;  // whole block
    const uint16_t *wm = sc.mat ? a.w1 : a.w0;
    void *ym = sc.mat ? a.y1 : a.y0;
    const __amdgpu_buffer_rsrc_t yr = out_rsrc(a, ym, M);

    {
        const __amdgpu_buffer_rsrc_t xs = make_rsrc(sc.mat ? a.x1 : a.x, x_bytes(a, M));
        const int ldx = a.ldx;
        auto src = [=](int i) {
            const int m = i / kvec;
            const int kv = i - m * kvec;
            return kv * 8 < K ? (unsigned)(m * ldx + kv * 8) * 2u : kOutOfRange;
        };
        u32x4 xt[kStageBatch];
        stage_issue(xs, M * kvec, src, xt);
        stage_finish(xs, M * kvec, src, xt, lds_x);
    }

    const int rows_t = (int)(blockDim.x >> 6) * R;
    for (int it = sc.first, t = sc.tile(it); t < a.tiles; it += sc.step, t = sc.tile(it)) {
        const int row0 = t * rows_t + wave * R;
        int valid = a.N - row0;
        valid = valid < 0 ? 0 : (valid > R ? R : valid);
        const __amdgpu_buffer_rsrc_t ws =
            make_rsrc(wm + (size_t)row0 * K, (unsigned)(valid * K * 2));

        float acc[M][R];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[m][r] = 0.0f;

        for (int k0 = 0; k0 < K; k0 += 512 * U) {
            u32x4 wv[R][U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + u * 512 + lane * 8;
#pragma unroll
                for (int r = 0; r < R; ++r)
                    wv[r][u] = load16<NT>(ws, k < K ? (unsigned)(r * K + k) * 2u : kOutOfRange);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kv = (k0 + u * 512) / 8 + lane;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const u32x4 xv = lds_x[m * kvec + kv];
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        acc[m][r] = dot8(wv[r][u], xv, acc[m][r]);
                }
            }
        }

#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r)
                acc[m][r] = group_sum<64>(acc[m][r]);

        // the sums sit in lane 63, lane 15 of the last 16-lane row
        store_results<M, R, 16>(a, yr, sum_lane<64>() - lane, [&](auto k, auto s) {
            return from_row_end<decltype(s)::value>(acc[k % M][k / M]);
        }, [&](int r) { return row0 + r; });
    }
}

// ---------------------------------------------------------------------------
// Family MFMA: the matrix cores do the multiplies.
//
// v_mfma_f32_4x4x4_16b_bf16 runs 16 independent 4x4x4 products per wave: block
// b = lanes 4b .. 4b+3, and lane (b, j) supplies row j of the block's A (4
// bfloat16), column j of its B, and holds column j of its 4x4 float32
// accumulator (one VGPR per row). Here A = x (row m, zero-cost padding for
// m >= M) and B = W^T (column j = output row j of a 4-row group), and the 16
// blocks take 16 consecutive 8-element K chunks of the same 4 rows. So lane
// (b, j) loads 16 bytes W[row j][k0 + 8b .. +8], which feed two MFMAs (k 0..3,
// then 4..7), and one load instruction reads 4 rows x 256 contiguous bytes.
// The A operand is x[m = j][the same 8 k], one 16-byte LDS read. Lanes j >= M
// read a valid x row: they only feed rows m >= M of the result, never stored.
// After the K loop the 16 block partials of each (m, row) are summed across
// lanes (DPP row rotations, then two cross-row shuffles), once per tile.
//
// A wave owns R groups of 4 rows; KW waves of a block split K and meet in LDS
// (fixed order). The K loop runs in batches of U loads per group; with PF the
// next batch (or the next tile's first batch) is loaded while the current one
// is multiplied. Requires K % (128 * KW) == 0 and (K / KW / 128) % U == 0.
// ---------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma4x4x4(unsigned a0, unsigned a1, unsigned b0, unsigned b1,
                                             f32x4_t c)
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, u32x2{a0, a1}),
                                                  __builtin_bit_cast(s16x4_t, u32x2{b0, b1}), c,
                                                  0, 0, 0);
}

template <int M, int U, int R, int KW, bool NT, bool PF>
__global__ __launch_bounds__(kMaxWaves * 64) void mfma_kernel(Args a)
{
    static_assert(M >= 1 && M <= 4, "the 4x4x4 MFMA's A operand holds 4 rows of x");
    extern __shared__ u32x4 mx_lds[];  // x as [M][K] bfloat16
    constexpr int ROWS_W = 4 * R;
    __shared__ float part[KW > 1 ? kMaxWaves * ROWS_W * M : 1];

    const int K = a.K;
    const int kslice = K / KW;
    const int nb = kslice / (128 * U);  // batches per tile
    const int groups = (int)(blockDim.x >> 6) / KW;
    const int rows_t = groups * ROWS_W;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kw = wave % KW;
    const int grp = wave / KW;
    const int lj = lane & 3;   // row of A / column of B and D within a block
    const int lb = lane >> 2;  // block: which 8-element K chunk
    const int xrow = lj < M ? lj : 0;
    const Sched sc = block_sched(a);
    const int step = sc.step;
    const uint16_t *wm = sc.mat ? a.w1 : a.w0;
    void *ym = sc.mat ? a.y1 : a.y0;
    const __amdgpu_buffer_rsrc_t yr = out_rsrc(a, ym, M);

    int it = sc.first;
    int tile = sc.tile(it);
    if (tile >= a.tiles)
        return;  // whole block

    // W loads of batch b of tile t for this wave's R groups (empty past the last tile).
    auto issue = [&](int t, int b, u32x4 (&wv)[R][U]) {
        const uint16_t *base = wm;
        int valid = 0;
        if (t < a.tiles) {
            const int row0 = t * rows_t + grp * ROWS_W;
            valid = a.N - row0;
            valid = valid < 0 ? 0 : (valid > ROWS_W ? ROWS_W : valid);
            base = wm + (size_t)row0 * K;
        }
        const __amdgpu_buffer_rsrc_t ws = make_rsrc(base, (unsigned)(valid * K * 2));
        const unsigned k0 = (unsigned)(kw * kslice + b * 128 * U + lb * 8);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int u = 0; u < U; ++u)
                wv[r][u] = load16<NT>(ws, ((unsigned)((r * 4 + lj) * K) + k0 + u * 128) * 2u);
    };

    u32x4 wa[R][U], wb[PF ? R : 1][PF ? U : 1];
    {
        // x pieces first (L2), then the weights (HBM), then x into LDS as [M][K]
        const __amdgpu_buffer_rsrc_t xs = make_rsrc(sc.mat ? a.x1 : a.x, x_bytes(a, M));
        const int ldx = a.ldx;
        const int kv8 = K / 8;
        auto src = [=](int i) {
            const int m = i / kv8;
            return (unsigned)(m * ldx + (i - m * kv8) * 8) * 2u;
        };
        u32x4 xt[kStageBatch];
        stage_issue(xs, M * kv8, src, xt);
        issue(tile, 0, wa);
        stage_finish(xs, M * kv8, src, xt, mx_lds);
    }

    f32x4_t acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto multiply = [&](int b, const u32x4 (&wv)[R][U]) {
        const int xk = kw * kslice + b * 128 * U + lb * 8;
        const volatile __attribute__((address_space(3))) u32x4 *xp =
            (const volatile __attribute__((address_space(3))) u32x4 *)mx_lds;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x4 xv = xp[(xrow * K + xk + u * 128) / 8];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                acc[r] = mfma4x4x4(xv[0], xv[1], wv[r][u][0], wv[r][u][1], acc[r]);
                acc[r] = mfma4x4x4(xv[2], xv[3], wv[r][u][2], wv[r][u][3], acc[r]);
            }
        }
    };

    // Sum the 16 block partials: lanes j, j+4, ..., j+60 hold the same (m, row).
    auto block_sum = [&](float v) {
        v = dpp_add<0x124>(v);  // row_ror:4
        v = dpp_add<0x128>(v);  // row_ror:8
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        return v;
    };

    auto finish = [&](int t) {
        const int row0 = t * rows_t + grp * ROWS_W;
        float s[R][M];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m)
                s[r][m] = block_sum(acc[r][m]);
        // every lane holds the sums of its row lj; block lb stores result lb
        auto row = [&](int r) { return row0 + r * 4 + lj; };
        if constexpr (KW == 1) {
            store_results<M, R, 16>(a, yr, lb, [&](auto k, auto) { return s[k / M][k % M]; }, row);
        } else {
            if (lb == 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < M; ++m)
                        part[((grp * KW + kw) * ROWS_W + r * 4 + lj) * M + m] = s[r][m];
            }
            __syncthreads();
            // the group's first wave sums and stores (a wave-uniform branch)
            if (kw == 0) {
                store_results<M, R, 16>(a, yr, lb, [&](auto k, auto) {
                    constexpr int m = decltype(k)::value % M, r = decltype(k)::value / M;
                    float v = part[((grp * KW + 0) * ROWS_W + r * 4 + lj) * M + m];
#pragma unroll
                    for (int q = 1; q < KW; ++q)
                        v += part[((grp * KW + q) * ROWS_W + r * 4 + lj) * M + m];
                    return v;
                }, row);
            }
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    };

    int b = 0;
    if constexpr (PF) {
        // One step: load the next batch into `nxt`, multiply `cur`, close the tile
        // after its last batch. Returns false when no step follows.
        auto run_step = [&](const u32x4 (&cur)[R][U], u32x4 (&nxt)[R][U]) {
            int t2 = tile, b2 = b + 1, it2 = it;
            if (b2 == nb) {
                b2 = 0;
                it2 = it + step;
                t2 = sc.tile(it2);
            }
            issue(t2, b2, nxt);
            multiply(b, cur);
            if (b + 1 == nb)
                finish(tile);
            tile = t2;
            it = it2;
            b = b2;
            return tile < a.tiles;
        };
        while (run_step(wa, wb) && run_step(wb, wa)) {
        }
    } else {
        while (true) {
            multiply(b, wa);
            if (++b == nb) {
                finish(tile);
                b = 0;
                it += step;
                tile = sc.tile(it);
                if (tile >= a.tiles)
                    break;
            }
            issue(tile, b, wa);
        }
    }
}

// ---------------------------------------------------------------------------
// Family SCALAR: any K, any alignment. One wave per output row (pair rows
// follow the first weight's rows), lanes stride K one element at a time,
// float32 fused multiply-add on exactly widened bfloat16 values.
// ---------------------------------------------------------------------------
template <int M>
__global__ __launch_bounds__(256) void scalar_kernel(Args a)
{
    const int lane = threadIdx.x & 63;
    const long long g = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= (long long)a.nmats * a.N)
        return;  // whole wave
    const int mat = g >= a.N ? 1 : 0;
    const int row = (int)(g - (long long)mat * a.N);
    const uint16_t *w = (mat ? a.w1 : a.w0) + (size_t)row * a.K;
    const uint16_t *xm = mat ? a.x1 : a.x;
    void *ym = mat ? a.y1 : a.y0;

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
        acc[m] = 0.0f;
    for (int k = lane; k < a.K; k += 64) {
        const float wf = bf16_to_f32(w[k]);
#pragma unroll
        for (int m = 0; m < M; ++m)
            acc[m] = __builtin_fmaf(bf16_to_f32(xm[(size_t)m * a.ldx + k]), wf, acc[m]);
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
        acc[m] = group_sum<64>(acc[m]);
    if (lane == sum_lane<64>()) {
#pragma unroll
        for (int m = 0; m < M; ++m)
            store_out(a, ym, (size_t)m * a.ldy + row, acc[m]);
    }
}

// K == 0: the empty sum, +0 for every (m, n) of y0 (and y1), rows at stride ldy;
// elements of `elem_bytes` (2 or 4) bytes.
[[maybe_unused]] static __global__ __launch_bounds__(256) void zero_kernel(
    void *y0, void *y1, int N, int ldy, long long count, int elem_bytes)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < count) {
        const long long m = i / N;
        const size_t o = (size_t)(m * ldy + (i - m * N));
        if (elem_bytes == 4) {
            static_cast<float *>(y0)[o] = 0.0f;
            if (y1)
                static_cast<float *>(y1)[o] = 0.0f;
        } else {
            static_cast<uint16_t *>(y0)[o] = 0;
            if (y1)
                static_cast<uint16_t *>(y1)[o] = 0;
        }
    }
}

}  // namespace skg
