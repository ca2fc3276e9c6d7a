// A C++ program that uses the library only through include/skinny_gemm.h: device
// memory from hipMalloc, inputs drawn on the host, one HIP stream, no Python and no
// torch. Each call's output is checked against the CPU oracle (oracle/skinny_oracle.c,
// linked in) with the acceptance rules of the Python tests: per element
// |y - y_ref| <= 1e-2 * sum_k |x_k W_nk| + 1e-6 and |y - ref64| <= 7.5e-5 + 2^-8 |ref64|,
// per output row cosine >= 0.99999. It also checks that invalid calls are refused
// with the documented status before anything runs, and that a graph captured around
// the calls replays them bit for bit; and exercises cross-block split-K with a
// hipMalloc workspace and on the library's static one.
//
// Built by tests/native/build_native.py (which __graft_entry__.build() calls) next to this file;
// run by tests/test_native_abi.py on a GPU. Exit status 0 = every check passed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "skinny_gemm.h"

extern "C" {
double oracle_bf16_to_f64(uint16_t h);
int oracle_gemm_bf16_rows(const uint16_t *x, const uint16_t *W, const int64_t *rows, int64_t nrows, int M, int K,
                          uint16_t *y, double *ref64, double *mag, double *x64, int nthreads);
}

namespace {

int failures = 0;

#define CHECK(cond, ...)                                                                                     \
    do {                                                                                                     \
        if (!(cond)) {                                                                                       \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);                                        \
            std::fprintf(stderr, __VA_ARGS__);                                                               \
            std::fprintf(stderr, "\n");                                                                      \
            ++failures;                                                                                      \
        }                                                                                                    \
    } while (0)

#define HIP_OK(expr)                                                                                         \
    do {                                                                                                     \
        const hipError_t e_ = (expr);                                                                        \
        if (e_ != hipSuccess) {                                                                              \
            std::fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__);     \
            std::exit(2);                                                                                    \
        }                                                                                                    \
    } while (0)

// Inputs: a 64-bit linear congruential stream turned into float32 normals by the
// Box-Muller transform, scaled, then rounded to bfloat16 to nearest even.
struct Rng {
    uint64_t s;
    double uniform()
    {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return ((s >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    }
    float normal()
    {
        const double u = uniform(), v = uniform();
        return (float)(std::sqrt(-2.0 * std::log(u)) * std::cos(6.283185307179586 * v));
    }
};

uint16_t to_bf16(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

std::vector<uint16_t> draw(size_t n, float scale, uint64_t seed)
{
    Rng r{seed * 0x9E3779B97F4A7C15ull + 1};
    std::vector<uint16_t> v(n);
    for (auto &e : v)
        e = to_bf16(r.normal() * scale);
    return v;
}

template <typename T>
T *to_device(const std::vector<T> &h)
{
    T *d = nullptr;
    HIP_OK(hipMalloc(&d, h.size() * sizeof(T)));
    HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}

// y: bfloat16 bits (f32 == false) or float32 values, [M][ldy] with the first N used.
void check(const char *what, const std::vector<uint16_t> &x, int ldx, const std::vector<uint16_t> &W, int M,
           int N, int K, const void *y_host, int ldy, bool f32)
{
    std::vector<uint16_t> xc((size_t)M * K);
    for (int m = 0; m < M; ++m)
        std::memcpy(&xc[(size_t)m * K], &x[(size_t)m * ldx], (size_t)K * 2);
    std::vector<uint16_t> yr((size_t)M * N);
    std::vector<double> ref((size_t)M * N), mag((size_t)M * N), x64((size_t)M * K);
    CHECK(oracle_gemm_bf16_rows(xc.data(), W.data(), nullptr, N, M, K, yr.data(), ref.data(), mag.data(),
                                x64.data(), 8) == 0,
          "%s: oracle refused", what);
    for (int m = 0; m < M; ++m) {
        double dot = 0, na = 0, nb = 0;
        for (int n = 0; n < N; ++n) {
            double v;
            if (f32)
                v = ((const float *)y_host)[(size_t)m * ldy + n];
            else
                v = oracle_bf16_to_f64(((const uint16_t *)y_host)[(size_t)m * ldy + n]);
            const size_t o = (size_t)m * N + n;
            const double yref = f32 ? ref[o] : oracle_bf16_to_f64(yr[o]);
            CHECK(std::fabs(v - yref) <= 1e-2 * mag[o] + 1e-6, "%s: G1 at (%d,%d): %g vs %g", what, m, n, v, yref);
            CHECK(std::fabs(v - ref[o]) <= 7.5e-5 + std::ldexp(std::fabs(ref[o]), -8), "%s: S1 at (%d,%d): %g vs %g",
                  what, m, n, v, ref[o]);
            dot += v * yref;
            na += v * v;
            nb += yref * yref;
        }
        const double cosine = (na == 0 && nb == 0) ? 1.0 : dot / std::sqrt(na * nb);
        CHECK(cosine >= 0.99999, "%s: row %d cosine %.9f", what, m, cosine);
    }
}

}  // namespace

int main()
{
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        std::fprintf(stderr, "no GPU\n");
        return 2;
    }
    HIP_OK(hipSetDevice(0));
    CHECK(skinny_gemm_init(0) == SKINNY_OK, "init");
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    // single calls: a ragged N over several tiles, every M, tuned and untuned shapes
    const int shapes[][2] = {{4096, 1024}, {1000, 1024}, {2048, 4096}, {300, 1536}, {77, 1000}};
    for (const auto &sh : shapes) {
        const int N = sh[0], K = sh[1];
        const auto W = draw((size_t)N * K, (float)(1.0 / std::sqrt((double)K)), (uint64_t)N * 131 + K);
        uint16_t *Wd = to_device(W);
        for (int M = 1; M <= 8; ++M) {
            const auto x = draw((size_t)M * K, 1.0f, (uint64_t)M * 7 + K);
            uint16_t *xd = to_device(x);
            uint16_t *yd = nullptr;
            float *y32d = nullptr;
            HIP_OK(hipMalloc(&yd, (size_t)M * N * 2));
            HIP_OK(hipMalloc(&y32d, (size_t)M * N * 4));
            CHECK(skinny_gemm_bf16(xd, Wd, yd, M, N, K, stream) == SKINNY_OK, "bf16 call M=%d N=%d K=%d", M, N, K);
            CHECK(skinny_gemm_bf16_f32out(xd, Wd, y32d, M, N, K, stream) == SKINNY_OK, "f32 call");
            HIP_OK(hipStreamSynchronize(stream));
            std::vector<uint16_t> y((size_t)M * N);
            std::vector<float> y32((size_t)M * N);
            HIP_OK(hipMemcpy(y.data(), yd, y.size() * 2, hipMemcpyDeviceToHost));
            HIP_OK(hipMemcpy(y32.data(), y32d, y32.size() * 4, hipMemcpyDeviceToHost));
            char what[96];
            std::snprintf(what, sizeof what, "bf16 (%d,%d) M=%d", N, K, M);
            check(what, x, K, W, M, N, K, y.data(), N, false);
            std::snprintf(what, sizeof what, "f32 (%d,%d) M=%d", N, K, M);
            check(what, x, K, W, M, N, K, y32.data(), N, true);
            HIP_OK(hipFree(xd));
            HIP_OK(hipFree(yd));
            HIP_OK(hipFree(y32d));
        }
        HIP_OK(hipFree(Wd));
    }

    // the paired forms: shared x, and two row-strided halves of a merged activation
    // into two halves of a merged output
    {
        const int N = 4096, K = 128, M = 4, ldx = 2 * K, ldy = 2 * N;
        const auto W0 = draw((size_t)N * K, (float)(1.0 / std::sqrt((double)K)), 11);
        const auto W1 = draw((size_t)N * K, (float)(1.0 / std::sqrt((double)K)), 12);
        const auto xm = draw((size_t)M * ldx, 1.0f, 13);
        uint16_t *W0d = to_device(W0), *W1d = to_device(W1), *xmd = to_device(xm);
        uint16_t *y0d = nullptr, *y1d = nullptr, *ymd = nullptr;
        HIP_OK(hipMalloc(&y0d, (size_t)M * N * 2));
        HIP_OK(hipMalloc(&y1d, (size_t)M * N * 2));
        HIP_OK(hipMalloc(&ymd, (size_t)M * ldy * 2));
        CHECK(skinny_gemm_bf16_pair_strided(xmd, xmd, ldx, W0d, W1d, y0d, y1d, N, M, N, K, stream) ==
                  SKINNY_OK,
              "pair on x0 = x1");
        CHECK(skinny_gemm_bf16_pair_strided(xmd, xmd + K, ldx, W0d, W1d, ymd, ymd + N, ldy, M, N, K, stream) ==
                  SKINNY_OK,
              "strided pair");
        HIP_OK(hipStreamSynchronize(stream));
        std::vector<uint16_t> y0((size_t)M * N), y1((size_t)M * N), ym((size_t)M * ldy);
        HIP_OK(hipMemcpy(y0.data(), y0d, y0.size() * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(y1.data(), y1d, y1.size() * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(ym.data(), ymd, ym.size() * 2, hipMemcpyDeviceToHost));
        check("pair y0", xm, ldx, W0, M, N, K, y0.data(), N, false);
        check("pair y1", xm, ldx, W1, M, N, K, y1.data(), N, false);
        std::vector<uint16_t> xh1(xm.begin() + K, xm.end());
        check("strided y0", xm, ldx, W0, M, N, K, ym.data(), ldy, false);
        check("strided y1", xh1, ldx, W1, M, N, K, ym.data() + N, ldy, false);

        // refused before anything runs: M out of range, a missing output, y over W,
        // the two outputs of a pair overlapping
        CHECK(skinny_gemm_bf16(xmd, W0d, y0d, 9, N, K, stream) == SKINNY_ERR_INVALID_ARG, "M = 9");
        CHECK(skinny_gemm_bf16(xmd, W0d, nullptr, 1, N, K, stream) == SKINNY_ERR_INVALID_ARG, "null y");
        CHECK(skinny_gemm_bf16(xmd, W0d, W0d, 1, N, K, stream) == SKINNY_ERR_INVALID_ARG, "y over W");
        CHECK(skinny_gemm_bf16_pair(xmd, W0d, W1d, y0d, y0d + 1, 1, N, K, stream) == SKINNY_ERR_INVALID_ARG,
              "overlapping pair outputs");
        CHECK(std::strlen(skinny_gemm_status_string(SKINNY_ERR_INVALID_ARG)) > 0, "status string");

        // a graph captured around the calls replays them bit for bit
        hipGraph_t graph;
        hipGraphExec_t exec;
        std::vector<uint16_t> e0 = y0;
        HIP_OK(hipMemsetAsync(y0d, 0, y0.size() * 2, stream));
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipStreamBeginCapture(stream, hipStreamCaptureModeGlobal));
        // the same call that produced e0: x rows at stride ldx
        CHECK(skinny_gemm_bf16_pair_strided(xmd, xmd, ldx, W0d, W1d, y0d, y1d, N, M, N, K, stream) == SKINNY_OK,
              "capture");
        HIP_OK(hipStreamEndCapture(stream, &graph));
        HIP_OK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
        for (int rep = 0; rep < 3; ++rep) {
            HIP_OK(hipMemsetAsync(y0d, 0xFF, y0.size() * 2, stream));
            HIP_OK(hipStreamSynchronize(stream));
            HIP_OK(hipGraphLaunch(exec, stream));
            HIP_OK(hipStreamSynchronize(stream));
            std::vector<uint16_t> g0((size_t)M * N);
            HIP_OK(hipMemcpy(g0.data(), y0d, g0.size() * 2, hipMemcpyDeviceToHost));
            CHECK(std::memcmp(g0.data(), e0.data(), g0.size() * 2) == 0, "graph replay %d", rep);
        }
        HIP_OK(hipGraphExecDestroy(exec));
        HIP_OK(hipGraphDestroy(graph));
        for (void *p : {(void *)W0d, (void *)W1d, (void *)xmd, (void *)y0d, (void *)y1d, (void *)ymd})
            HIP_OK(hipFree(p));
    }
    // cross-block split-K: a workspace from hipMalloc, zeroed once and reused across
    // shapes, and the library's static workspace; both against the oracle and each other
    {
        const size_t ws_bytes = skinny_gemm_split_k_workspace_bytes(8, 4096, 8192, nullptr);
        CHECK(ws_bytes > 0, "workspace size");
        void *ws = nullptr;
        HIP_OK(hipMalloc(&ws, ws_bytes));
        HIP_OK(hipMemset(ws, 0, ws_bytes));
        const int sk_shapes[][3] = {{4096, 8192, 4}, {2048, 4096, 1}, {1000, 4096, 8}, {8192, 1536, 2}};
        for (const auto &sh : sk_shapes) {
            const int N = sh[0], K = sh[1], M = sh[2];
            CHECK(skinny_gemm_split_k_workspace_bytes(M, N, K, nullptr) <= ws_bytes, "fits");
            const auto W = draw((size_t)N * K, (float)(1.0 / std::sqrt((double)K)), (uint64_t)N * 7 + K);
            const auto x = draw((size_t)M * K, 1.0f, (uint64_t)M * 11 + K);
            uint16_t *Wd = to_device(W), *xd = to_device(x), *y1 = nullptr, *y2 = nullptr;
            HIP_OK(hipMalloc(&y1, (size_t)M * N * 2));
            HIP_OK(hipMalloc(&y2, (size_t)M * N * 2));
            CHECK(skinny_gemm_bf16_split_k(xd, Wd, y1, M, N, K, nullptr, ws, ws_bytes, stream) == SKINNY_OK,
                  "split-K (%d,%d) M=%d", N, K, M);
            CHECK(skinny_gemm_bf16_split_k_noalloc(xd, Wd, y2, M, N, K, nullptr, stream) == SKINNY_OK,
                  "split-K no-alloc (%d,%d) M=%d", N, K, M);
            HIP_OK(hipStreamSynchronize(stream));
            std::vector<uint16_t> h1((size_t)M * N), h2((size_t)M * N);
            HIP_OK(hipMemcpy(h1.data(), y1, h1.size() * 2, hipMemcpyDeviceToHost));
            HIP_OK(hipMemcpy(h2.data(), y2, h2.size() * 2, hipMemcpyDeviceToHost));
            char what[96];
            std::snprintf(what, sizeof what, "split-K (%d,%d) M=%d", N, K, M);
            check(what, x, K, W, M, N, K, h1.data(), N, false);
            CHECK(std::memcmp(h1.data(), h2.data(), h1.size() * 2) == 0, "no-alloc bits (%d,%d) M=%d", N, K, M);
            for (void *p : {(void *)Wd, (void *)xd, (void *)y1, (void *)y2})
                HIP_OK(hipFree(p));
        }
        // refused before anything runs: too small a workspace, the static one exceeded
        CHECK(skinny_gemm_bf16_split_k(nullptr, nullptr, nullptr, 1, 4096, 4096, nullptr, ws, 1024, stream) ==
                  SKINNY_ERR_INVALID_ARG,
              "null inputs");
        HIP_OK(hipFree(ws));
    }
    HIP_OK(hipStreamDestroy(stream));
    std::printf("abi_native: library version %d, %d variants, %d failures\n", skinny_gemm_version(),
                skinny_gemm_num_variants(), failures);
    return failures == 0 ? 0 : 1;
}
