// Sanitizer driver for the C ABI's host-side argument checks
// (bf16_skinny_gemm_amd/csrc/validate.hpp), built with g++
// -fsanitize=address,undefined on the CPU by tests/test_sanitizers.py.
//
// Random calls over a small fake address space (pointers are never
// dereferenced): whenever validate() accepts a call, no byte the kernels write
// (the M rows of y, and of y1 for a pair) may coincide with a byte they read
// (the rows of x / x1, all of W / W1), and the two outputs of a pair may not
// share a byte, checked byte by byte; the strided-pair test must also accept
// every pair of output views that is in fact disjoint. Then large and extreme
// sizes (up to INT_MAX, pointers up to 2^47) run through every check so that
// the undefined-behaviour sanitizer sees the overflow-prone arithmetic. The
// split-K checks (plan fields, workspace layout, a caller's workspace) run the
// same way.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "validate.hpp"

using namespace skg_host;

static unsigned long long g_state = 0x9E3779B97F4A7C15ull;
static unsigned long long next_u64()
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return g_state;
}
static int rnd(int lo, int hi) { return lo + (int)(next_u64() % (unsigned long long)(hi - lo + 1)); }

static int failures = 0;
#define EXPECT(cond, ...)                                                                           \
    do {                                                                                            \
        if (!(cond)) {                                                                              \
            std::fprintf(stderr, __VA_ARGS__);                                                      \
            std::fprintf(stderr, "\n");                                                             \
            if (++failures > 20)                                                                    \
                std::exit(1);                                                                       \
        }                                                                                           \
    } while (0)

using Bytes = std::set<uintptr_t>;

static void add_rows(Bytes &b, const void *p, int rows, int width, int stride, int elem)
{
    if (!p)
        return;
    const uintptr_t base = reinterpret_cast<uintptr_t>(p);
    for (int r = 0; r < rows; ++r)
        for (int i = 0; i < width * elem; ++i)
            b.insert(base + ((uintptr_t)r * stride) * elem + i);
}

static bool meet(const Bytes &a, const Bytes &b)
{
    for (uintptr_t v : a)
        if (b.count(v))
            return true;
    return false;
}

static const void *fake(uintptr_t base, int span)
{
    if (rnd(0, 15) == 0)
        return nullptr;
    uintptr_t off = (uintptr_t)rnd(0, span);
    if (rnd(0, 7) != 0)
        off &= ~(uintptr_t)(rnd(0, 1) ? 15 : 1);  // mostly 2- or 16-byte aligned
    return reinterpret_cast<const void *>(base + off);
}

int main()
{
    const uintptr_t base = 0x100000;
    long accepted = 0, pairs_disjoint = 0;
    for (int it = 0; it < 200000; ++it) {
        Call c{};
        c.M = rnd(-1, 9);
        c.N = rnd(-1, 6);
        c.K = rnd(-1, 6);
        c.nmats = rnd(1, 2);
        c.ldx = c.K + rnd(-1, 3);
        c.ldy = c.N + rnd(-1, 3);
        c.out_f32 = rnd(0, 1);
        const int arena = 400;
        c.x = fake(base, arena);
        c.x1 = c.nmats == 2 ? fake(base, arena) : c.x;
        c.w0 = fake(base, arena);
        c.w1 = c.nmats == 2 ? fake(base, arena) : nullptr;
        c.y0 = const_cast<void *>(fake(base, arena));
        c.y1 = c.nmats == 2 ? const_cast<void *>(fake(base, arena)) : nullptr;
        const int st = validate(c);
        EXPECT(st == SKINNY_OK || st == SKINNY_ERR_INVALID_ARG, "status %d", st);
        const int ye = c.out_f32 ? 4 : 2;
        if (st == SKINNY_OK && c.M > 0 && c.N > 0) {
            ++accepted;
            Bytes in, out0, out1;
            if (c.K > 0) {
                add_rows(in, c.x, c.M, c.K, c.ldx, 2);
                add_rows(in, c.w0, c.N, c.K, c.K, 2);
                if (c.nmats == 2) {
                    add_rows(in, c.x1, c.M, c.K, c.ldx, 2);
                    add_rows(in, c.w1, c.N, c.K, c.K, 2);
                }
            }
            add_rows(out0, c.y0, c.M, c.N, c.ldy, ye);
            add_rows(out1, c.y1, c.M, c.N, c.ldy, ye);
            EXPECT(!meet(out0, in) && !meet(out1, in), "accepted an output over an input (it %d)", it);
            EXPECT(!meet(out0, out1), "accepted overlapping pair outputs (it %d)", it);
            const void *ps[6] = {c.x, c.x1, c.w0, c.w1, c.y0, c.y1};
            for (const void *p : ps)
                EXPECT(!p || reinterpret_cast<uintptr_t>(p) % 2 == 0, "accepted an odd pointer");
            if (c.out_f32)
                EXPECT(reinterpret_cast<uintptr_t>(c.y0) % 4 == 0, "accepted a misaligned float32 output");
            if (c.K > 0 && vector_ok(c)) {
                EXPECT(reinterpret_cast<uintptr_t>(c.x) % 16 == 0 && reinterpret_cast<uintptr_t>(c.w0) % 16 == 0 &&
                           c.K % 8 == 0 && c.ldx % 8 == 0,
                       "vector path for a misaligned call");
            }
            (void)out_span_ok(c);
        }
        // the strided-pair test is exact: disjoint row sets are always accepted
        if (c.nmats == 2 && c.M > 0 && c.N > 0 && c.ldy >= c.N && c.y0 && c.y1) {
            Bytes a, b;
            add_rows(a, c.y0, c.M, c.N, c.ldy, ye);
            add_rows(b, c.y1, c.M, c.N, c.ldy, ye);
            const bool disjoint = !meet(a, b);
            pairs_disjoint += disjoint;
            EXPECT(strided_disjoint(c.y0, c.y1, c.M, (size_t)c.N * ye, (size_t)c.ldy * ye) == disjoint,
                   "strided_disjoint wrong: M %d N %d ldy %d elem %d", c.M, c.N, c.ldy, ye);
        }
    }

    // extreme sizes: every check runs, nothing may overflow (the sanitizer watches)
    const int edges[] = {0, 1, 7, 8, 9, 4096, (1 << 20) - 8, 1 << 20, (1 << 20) + 8, (1 << 30), INT_MAX - 7, INT_MAX};
    const uintptr_t ptrs[] = {0, 2, 16, 0x7FFFFFFFF000ull, 0x7FFFFFFFFFF0ull};
    long extreme = 0;
    for (int N : edges)
        for (int K : edges)
            for (int M = 0; M <= 9; ++M)
                for (int nm = 1; nm <= 2; ++nm)
                    for (int f32 = 0; f32 <= 1; ++f32) {
                        Call c{};
                        c.M = M;
                        c.N = N;
                        c.K = K;
                        c.nmats = nm;
                        c.out_f32 = f32;
                        c.ldx = K + (int)(next_u64() % 2) * (K < INT_MAX - 8 ? 8 : 0);
                        c.ldy = N;
                        c.x = reinterpret_cast<const void *>(ptrs[next_u64() % 5]);
                        c.x1 = nm == 2 ? reinterpret_cast<const void *>(ptrs[next_u64() % 5]) : c.x;
                        c.w0 = reinterpret_cast<const void *>(ptrs[next_u64() % 5]);
                        c.w1 = nm == 2 ? reinterpret_cast<const void *>(ptrs[next_u64() % 5]) : nullptr;
                        c.y0 = reinterpret_cast<void *>(ptrs[next_u64() % 5]);
                        c.y1 = nm == 2 ? reinterpret_cast<void *>(ptrs[next_u64() % 5]) : nullptr;
                        if (validate(c) == SKINNY_OK && M > 0 && N > 0 && K > 0) {
                            ++extreme;
                            if (vector_ok(c) && out_span_ok(c)) {
                                const uint64_t k = cache_key(3, c);
                                EXPECT(k >> 63 == 1, "cache key without its top bit");
                            }
                        }
                    }

    // cache keys are distinct for distinct (device, pair, M, K, N) on the vector path
    std::set<uint64_t> keys;
    long nkeys = 0;
    for (int dev : {0, 1, 63})
        for (int nm = 1; nm <= 2; ++nm)
            for (int M = 1; M <= kMaxM; ++M)
                for (int K : {8, 128, 4096, 1 << 20})
                    for (int N : {1, 2, 4096, 77440, INT_MAX}) {
                        Call c{};
                        c.M = M;
                        c.N = N;
                        c.K = K;
                        c.nmats = nm;
                        keys.insert(cache_key(dev, c));
                        ++nkeys;
                    }
    EXPECT((long)keys.size() == nkeys, "cache key collision: %zu distinct of %ld", keys.size(), nkeys);

    // cross-block split-K: plan fields, layout and a caller's workspace. When the
    // checks accept a call, the workspace bytes the kernel touches (counters, then
    // partials) share no byte with x, W or y, lie inside the given workspace, and the
    // tiles cover N exactly; random plan fields are accepted only inside their ranges.
    long split_accepted = 0;
    for (int it = 0; it < 20000; ++it) {
        const int M = rnd(1, kMaxM), N = rnd(1, 600), K = 8 * rnd(1, 64);
        const uintptr_t x = 0x10000 + 16 * (uintptr_t)rnd(0, 4096), w = 0x40000 + 16 * (uintptr_t)rnd(0, 4096);
        const uintptr_t y = 0x30000 + 2 * (uintptr_t)rnd(0, 65536);
        // now and then a workspace off its 256-byte alignment, which must be refused
        const uintptr_t ws = 256 * (uintptr_t)rnd(1, 4096) + (rnd(0, 15) == 0 ? 16 : 0);
        auto ptr = [](uintptr_t a) { return reinterpret_cast<void *>(a); };
        const Call c = single_call(ptr(x), ptr(w), ptr(y), M, N, K, 0);
        skinny_plan_t p{SKINNY_KIND_SPLIT_K, 64 * rnd(0, 10), 64, 1, 1, rnd(0, 70), rnd(0, 1), rnd(0, 1) * rnd(0, 4),
                        rnd(0, 1) * rnd(0, 2), rnd(0, 1) * rnd(0, 2)};
        const bool fields = split_fields_ok(p);
        EXPECT(fields == (p.threads_per_block >= 64 && p.threads_per_block <= 512 && p.k_split >= 1 &&
                          p.k_split <= 64 && p.nontemporal == 1 && p.grid_blocks == 0 && p.x_in_lds == 0 &&
                          p.prefetch == 0),
               "split fields decision");
        if (!fields || validate(c) != SKINNY_OK || !split_call_ok(c))
            continue;
        const int rows_group = rnd(1, 4);
        const SplitLayout l = split_layout(p.threads_per_block, rows_group, p.k_split, M, N);
        const long long rows_t = (long long)(p.threads_per_block / 64) * rows_group;
        EXPECT(l.tiles * rows_t >= N && (l.tiles - 1) * rows_t < N, "tiles do not cover N");
        EXPECT(l.total == kSplitPartOffset + (size_t)p.k_split * M * N * 4, "layout size");
        const size_t given = l.total + (size_t)rnd(-64, 64) * 4;
        if (!split_layout_ok(l, p.k_split) || !split_workspace_ok(c, ptr(ws), given, l))
            continue;
        ++split_accepted;
        EXPECT(given >= l.total && ws % 256 == 0, "accepted a small or misaligned workspace");
        const uintptr_t lo = ws, hi = ws + l.total;
        auto meets = [&](uintptr_t b, size_t n) { return n > 0 && b < hi && lo < b + n; };
        EXPECT(!meets(x, span(M, K, K, 2)) && !meets(w, (size_t)N * K * 2) && !meets(y, (size_t)M * N * 2),
               "accepted a workspace that meets x, W or y");
        EXPECT(kSplitPartOffset >= (size_t)l.tiles * 4, "counters run into the partials");
    }
    // extreme sizes through the layout arithmetic (for the undefined-behaviour sanitizer)
    for (int N : {1, 65536, 1 << 20, INT_MAX})
        for (int S : {1, 16, 64})
            for (int t : {64, 512}) {
                const SplitLayout l = split_layout(t, 4, S, kMaxM, N);
                EXPECT(l.tiles >= 1 && l.total > l.part_bytes, "extreme layout");
                (void)split_layout_ok(l, S);
            }

    std::printf("validate_fuzz: %ld accepted random calls, %ld disjoint pair views, %ld extreme calls "
                "accepted, %ld cache keys, %ld split-K workspaces accepted, %d failures\n",
                accepted, pairs_disjoint, extreme, nkeys, split_accepted, failures);
    return failures == 0 ? 0 : 1;
}
