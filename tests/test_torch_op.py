"""The torch custom op and module hook (routing layer above the C ABI)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.fixture(scope="module")
def op():
    from bf16_skinny_gemm_amd.build import LIB_PATH
    import os

    from bf16_skinny_gemm_amd.build import TORCH_OP_PATH

    if not os.path.exists(LIB_PATH) or not os.path.exists(TORCH_OP_PATH):
        import __graft_entry__

        __graft_entry__.build()
    from bf16_skinny_gemm_amd import torch_op

    return torch_op


def test_cpu_tensors_route_to_fallback_or_raise(op):
    x = torch.randn(2, 16, dtype=torch.bfloat16)
    w = torch.randn(8, 16, dtype=torch.bfloat16)
    assert not op.qualifies(x, w)
    y = op.skinny_linear(x, w)
    assert torch.equal(y, torch.nn.functional.linear(x, w))
    with pytest.raises(ValueError):
        op.skinny_linear(x, w, fallback=False)
    with pytest.raises(ValueError):
        torch.ops.skinny.linear(x, w)


def test_cpp_registration_when_built(op):
    """With libskinny_torch_op.so built, the operator's kernels are the C++ ones:
    the schema comes from it and a CPU call raises its ValueError."""
    import os

    from bf16_skinny_gemm_amd.build import TORCH_OP_PATH

    assert op.CPP_OP == os.path.exists(TORCH_OP_PATH)
    if not op.CPP_OP:
        pytest.skip("the C++ operator library is not built")
    assert str(torch.ops.skinny.linear.default._schema) == "skinny::linear(Tensor x, Tensor weight) -> Tensor"
    with pytest.raises(ValueError, match="gfx950 GPU tensors only"):
        torch.ops.skinny.linear(torch.zeros(1, 8, dtype=torch.bfloat16), torch.zeros(4, 8, dtype=torch.bfloat16))


def test_fake_impl_shapes(op):
    x = torch.empty(1, 3, 64, dtype=torch.bfloat16, device="meta")
    w = torch.empty(40, 64, dtype=torch.bfloat16, device="meta")
    y = torch.ops.skinny.linear(x, w)
    assert y.shape == (1, 3, 40) and y.device.type == "meta"


@pytest.mark.gpu
def test_op_runs_the_kernel(op):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bf16_skinny_gemm_amd as skg

    N, K = 4096, 1024
    W = synth.weights(N, K, seed=130)
    Wd = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).cuda()
    for shape in ((1, K), (3, K), (1, 4, K), (2, 2, K)):
        M = int(np.prod(shape[:-1]))
        x = synth.activations(M, K, seed=131, tensor_id=M)
        xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda().reshape(shape)
        assert op.qualifies(xd, Wd)
        y = torch.ops.skinny.linear(xd, Wd)
        torch.cuda.synchronize()
        assert y.shape == (*shape[:-1], N)
        ref = skg.gemm(xd.reshape(M, K), Wd)
        assert torch.equal(y.reshape(M, N).view(torch.int16), ref.view(torch.int16))
        yb = y.reshape(M, N).view(torch.int16).cpu().numpy().view(np.uint16)
        yr, r64, mag = oracle.gemm(x, W)
        assert oracle.acceptance(yb, yr, r64, mag)["pass"]


@pytest.mark.gpu
def test_module_hook_and_routing(op):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.manual_seed(0)
    model = torch.nn.Sequential(torch.nn.Linear(512, 1024, bias=False),
                                torch.nn.Linear(1024, 256, bias=False),
                                torch.nn.Linear(256, 64, bias=True)).cuda().to(torch.bfloat16)
    x = torch.randn(2, 512, device="cuda").to(torch.bfloat16)
    ref = [x]
    for layer in model:
        ref.append(torch.nn.functional.linear(ref[-1], layer.weight, layer.bias))
    assert op.install(model) == 3
    y = model(x)
    torch.cuda.synchronize()
    # the bias-free layers ran the skinny GEMM, the biased one F.linear; compare in float32
    h1 = torch.ops.skinny.linear(x, model[0].weight)
    h2 = torch.ops.skinny.linear(h1, model[1].weight)
    h3 = torch.nn.functional.linear(h2, model[2].weight, model[2].bias)
    assert torch.equal(y, h3)
    assert torch.allclose(y.float(), ref[-1].float(), rtol=0.05, atol=0.05)
    # M = 8 still takes the skinny GEMM; M = 9 is outside its range: routed to F.linear,
    # or refused without fallback
    x8 = torch.randn(8, 512, device="cuda").to(torch.bfloat16)
    assert op.qualifies(x8, model[0].weight)
    assert torch.equal(op.skinny_linear(x8, model[0].weight),
                       torch.ops.skinny.linear(x8, model[0].weight))
    x9 = torch.randn(9, 512, device="cuda").to(torch.bfloat16)
    assert not op.qualifies(x9, model[0].weight)
    assert torch.equal(op.skinny_linear(x9, model[0].weight),
                       torch.nn.functional.linear(x9, model[0].weight))
    with pytest.raises(ValueError):
        op.skinny_linear(x9, model[0].weight, fallback=False)


@pytest.mark.gpu
def test_op_under_graph_capture(op):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = torch.randn(2048, 4096, device="cuda").to(torch.bfloat16)
    x = torch.randn(4, 4096, device="cuda").to(torch.bfloat16)
    eager = torch.ops.skinny.linear(x, w)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        torch.ops.skinny.linear(x, w)
        with torch.cuda.graph(g, stream=s):
            out = torch.ops.skinny.linear(x, w)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))


@pytest.mark.gpu
def test_strided_weight_is_not_routed(op):
    """A non-contiguous weight would need a whole copy per call: it stays on F.linear."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.manual_seed(1)
    wt = torch.randn(512, 256, device="cuda").to(torch.bfloat16)
    w = wt.t()  # [256, 512] view with strides (1, 256)
    x = torch.randn(2, 512, device="cuda").to(torch.bfloat16)
    assert not w.is_contiguous()
    assert not op.qualifies(x, w)
    assert torch.equal(op.skinny_linear(x, w), torch.nn.functional.linear(x, w))
    with pytest.raises(ValueError):
        torch.ops.skinny.linear(x, w)


@pytest.mark.gpu
def test_op_under_torch_compile(op):
    """The op traces (its fake implementation gives the output metadata) and the
    compiled function runs the same kernel: same bits as the eager call."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.manual_seed(2)
    w = (torch.randn(4096, 1024, device="cuda") / 32).to(torch.bfloat16)
    x = torch.randn(2, 3, 1024, device="cuda").to(torch.bfloat16)

    def f(a, b):
        return torch.ops.skinny.linear(a, b) * 2

    compiled = torch.compile(f, backend="aot_eager", fullgraph=True)
    y = compiled(x, w)
    torch.cuda.synchronize()
    assert y.shape == (2, 3, 4096)
    assert torch.equal(y.view(torch.int16), f(x, w).view(torch.int16))
