// torch.ops.skinny.linear with its GPU kernel registered in C++: the eager call
// goes from the dispatcher straight to the C ABI (include/skinny_gemm.h), with no
// Python frame in between. vLLM PR #65306 (SM90 skinny GEMM plans), section
// Details, puts the eager overhead of its custom op at 4-7 us per call; the C ABI
// call alone costs about 4 us here (almost all of it HIP's kernel launch), and
// this registration adds the dispatcher and the output allocation to it.
//
// Only argument marshalling lives here: shape, dtype and device checks, the
// output tensor, the current HIP stream. The product runs in the HIP kernels.
// The fake (meta) implementation used for tracing is registered from Python
// (bf16_skinny_gemm_amd/torch_op.py), which this library names as the op's
// Python module.
#include <ATen/core/Tensor.h>
#include <ATen/ops/empty.h>
#include <c10/core/DeviceGuard.h>
#include <c10/hip/HIPStream.h>
#include <torch/library.h>

#include <climits>

#include "skinny_gemm.h"

namespace {

// y[..., N] = x[..., K] . weight[N, K]^T for bfloat16 x with prod(leading dims) = M
// in 1..8 and a contiguous bfloat16 weight on the same GPU. Refusals raise
// ValueError (the calls a router should have sent elsewhere); a refusal by the
// library itself (not gfx950, launch failure) raises RuntimeError.
at::Tensor linear_gpu(const at::Tensor &x, const at::Tensor &weight)
{
    TORCH_CHECK_VALUE(x.scalar_type() == at::kBFloat16 && weight.scalar_type() == at::kBFloat16,
                      "skinny::linear: x and weight must be bfloat16, got ", x.scalar_type(), " and ",
                      weight.scalar_type());
    TORCH_CHECK_VALUE(x.device() == weight.device(), "skinny::linear: x on ", x.device(), ", weight on ",
                      weight.device());
    TORCH_CHECK_VALUE(weight.dim() == 2 && x.dim() >= 1 && x.size(-1) == weight.size(1),
                      "skinny::linear: shapes x ", x.sizes(), " and weight ", weight.sizes(), " do not match");
    TORCH_CHECK_VALUE(weight.is_contiguous(), "skinny::linear: weight must be contiguous");
    const int64_t K = x.size(-1), N = weight.size(0);
    const int64_t M = K > 0 ? x.numel() / K : 0;
    TORCH_CHECK_VALUE(M >= 1 && M <= 8 && x.numel() == M * K,
                      "skinny::linear: the token count prod(x.shape[:-1]) must be 1..8, got x ", x.sizes());
    TORCH_CHECK_VALUE(N <= INT_MAX && K <= INT_MAX, "skinny::linear: N and K must fit in 32 bits");

    c10::DeviceGuard guard(x.device());
    const at::Tensor x2 = x.reshape({M, K}).contiguous();
    std::vector<int64_t> shape(x.sizes().begin(), x.sizes().end());
    shape.back() = N;
    at::Tensor y = at::empty(shape, x.options());
    const hipStream_t stream = c10::hip::getCurrentHIPStream(x.device().index()).stream();
    const int st = skinny_gemm_bf16(x2.data_ptr(), weight.data_ptr(), y.data_ptr(), (int)M, (int)N, (int)K, stream);
    TORCH_CHECK(st == SKINNY_OK, "skinny::linear: skinny_gemm_bf16 returned ", st, " (",
                skinny_gemm_status_string(st), ")");
    return y;
}

at::Tensor linear_cpu(const at::Tensor &x, const at::Tensor &weight)
{
    TORCH_CHECK_VALUE(false, "skinny::linear: runs on gfx950 GPU tensors only, got x on ", x.device(),
                      ", weight on ", weight.device());
    return at::Tensor();
}

}  // namespace

TORCH_LIBRARY(skinny, m)
{
    m.set_python_module("bf16_skinny_gemm_amd.torch_op");
    m.def("linear(Tensor x, Tensor weight) -> Tensor");
}

TORCH_LIBRARY_IMPL(skinny, CUDA, m) { m.impl("linear", &linear_gpu); }

TORCH_LIBRARY_IMPL(skinny, CPU, m) { m.impl("linear", &linear_cpu); }
