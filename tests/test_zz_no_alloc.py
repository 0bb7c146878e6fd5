"""grpo_loss_fwd_noalloc (the forward with its scratch in a static device
array) against grpo_loss_fwd with a caller's workspace, through the C ABI:
the same kernels on the same inputs, so every output must be bitwise equal.
Two calls in a row, the second on a smaller input (the static scratch keeps
the first call's contents), in float32 and bfloat16, and a shape whose
scratch would exceed the static array is refused on the host."""
import ctypes

import pytest
import torch

import workloads
from tests.gpu_common import BETA, EPS

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("grpo_policy_loss_amd")


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _case(w, seed):
    inp = workloads.generate(w, seed=seed, device="cuda")
    adv = gp.grpo_advantages(inp["rewards"], w.G, EPS)
    ref = gp.grpo_ref_logprobs(inp["H_ref"], inp["W"], inp["y"], w.chunk)
    want = gp.grpo_loss_fwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref, w.B, w.L, BETA,
                            w.chunk)
    return inp, adv, ref, want


def _noalloc(w, inp, adv, ref, opts=None):
    dt = gp.GRPO_F32 if w.dtype == "f32" else gp.GRPO_BF16
    loss = torch.full((1,), float("nan"), device="cuda")
    lp, kl, lse = (torch.full((w.N,), float("nan"), device="cuda") for _ in range(3))
    st = gp.lib().grpo_loss_fwd_noalloc(
        _p(inp["H"]), _p(inp["W"]), _p(inp["y"]), _p(inp["mask"]), _p(adv), _p(ref), w.B, w.L,
        w.d, w.V, dt, BETA, w.chunk, gp._lib._opts(opts), _p(loss), _p(lp), _p(kl), _p(lse),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, gp.lib().grpo_last_error().decode()
    return loss, lp, kl, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_forward_equals_the_workspace_forward_twice(dtype):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    base = workloads.WORKLOADS[0]
    big = base.scaled(name="na-big", prompts=2, G=3, L=700, d=320, V=3000, dtype=dtype,
                      chunk=1024, len_lo=100, len_hi=700)
    small = base.scaled(name="na-small", prompts=1, G=3, L=100, d=256, V=1000, dtype=dtype,
                        chunk=256, len_lo=30, len_hi=100)
    for w, seed in ((big, 41), (small, 42)):
        print(f"[noalloc] {dtype} {w.name} N={w.N} V={w.V} chunk={w.chunk}", flush=True)
        inp, adv, ref, want = _case(w, seed)
        got = _noalloc(w, inp, adv, ref)
        torch.cuda.synchronize()
        for name, g, e in zip(("loss", "lp", "kl", "lse"), got, want):
            assert torch.equal(g, e), name


def test_noalloc_forward_with_options_and_size_limit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = workloads.WORKLOADS[0].scaled(name="na-opts", prompts=2, G=2, L=300, d=64, V=700,
                                      dtype="bf16", chunk=256, len_lo=50, len_hi=300)
    opts = {"logit_softcapping": 20.0, "temperature": 0.8, "kl_estimator": 1, "aggregation": 1}
    inp = workloads.generate(w, seed=43, device="cuda")
    adv = gp.grpo_advantages(inp["rewards"], w.G, EPS)
    ref = gp.grpo_ref_logprobs(inp["H_ref"], inp["W"], inp["y"], w.chunk, opts=opts)
    want = gp.grpo_loss_fwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref, w.B, w.L, BETA,
                            w.chunk, opts=opts)
    got = _noalloc(w, inp, adv, ref, opts)
    torch.cuda.synchronize()
    for name, g, e in zip(("loss", "lp", "kl", "lse"), got, want):
        assert torch.equal(g, e), name
    # a shape whose scratch exceeds the static array: refused before any launch
    one = ctypes.c_void_p(16)
    st = gp.lib().grpo_loss_fwd_noalloc(one, one, one, one, one, one, 8, 4096, 1536, 151936, 1,
                                        BETA, 16384, None, one, one, one, one, None)
    assert st == -2
    assert b"static scratch" in gp.lib().grpo_last_error()
