"""The Python binding checks every tensor's dtype and size before it calls
the C ABI (which sees only pointers and cannot): a dH or dW of the wrong
shape or dtype, a short output, or index/mask/per-token vectors of the wrong
type would otherwise be read or written past their end on the GPU.  CPU
tensors are enough here: each bad argument is rejected, naming it, before
the device check or any library call."""
import pytest
import torch

gp = pytest.importorskip("grpo_policy_loss_amd")

N, B, L, d, V = 12, 3, 4, 16, 40


def _args(dtype=torch.bfloat16):
    return dict(H=torch.zeros(N, d, dtype=dtype), W=torch.zeros(V, d, dtype=dtype),
                y=torch.zeros(N, dtype=torch.int32), mask=torch.ones(N, dtype=torch.uint8),
                adv=torch.zeros(B), ref_lp=torch.zeros(N), lp=torch.zeros(N), lse=torch.zeros(N))


def _bwd(**over):
    a = _args()
    a.update(over)
    return gp.grpo_loss_bwd(a["H"], a["W"], a["y"], a["mask"], a["adv"], a["ref_lp"], a["lp"],
                            a["lse"], B, L, dW=a.get("dW"), dH=a.get("dH"))


def _fwd(**over):
    a = _args()
    a.update(over)
    return gp.grpo_loss_fwd(a["H"], a["W"], a["y"], a["mask"], a["adv"], a["ref_lp"], B, L)


def test_valid_arguments_reach_the_device_check():
    with pytest.raises(ValueError, match="on the GPU"):
        _bwd()
    with pytest.raises(ValueError, match="on the GPU"):
        _fwd()


@pytest.mark.parametrize("over,err,what", [
    ({"dH": torch.zeros(N, d, dtype=torch.float32)}, TypeError, "dH"),        # f32 dH for bf16 H
    ({"dH": torch.zeros(N - 1, d, dtype=torch.bfloat16)}, ValueError, "dH"),
    ({"dW": torch.zeros(V, d + 8)}, ValueError, "dW"),
    ({"dW": torch.zeros(d, V)}, ValueError, "dW"),
    ({"dW": torch.zeros(V, d, dtype=torch.bfloat16)}, TypeError, "dW"),
    ({"y": torch.zeros(N, dtype=torch.int64)}, TypeError, "y"),
    ({"y": torch.zeros(N - 1, dtype=torch.int32)}, ValueError, "y"),
    ({"mask": torch.ones(N, dtype=torch.bool)}, TypeError, "mask"),
    ({"adv": torch.zeros(B + 1)}, ValueError, "adv"),
    ({"lp": torch.zeros(N, dtype=torch.float64)}, TypeError, "lp"),
    ({"lse": torch.zeros(N + 1)}, ValueError, "lse"),
    ({"ref_lp": torch.zeros(N - 2)}, ValueError, "ref_lp"),
    ({"W": torch.zeros(V, d, dtype=torch.float32)}, TypeError, "W"),
    ({"W": torch.zeros(V, d + 8, dtype=torch.bfloat16)}, ValueError, "W"),
])
def test_backward_rejects_bad_arguments(over, err, what):
    with pytest.raises(err, match=what):
        _bwd(**over)


@pytest.mark.parametrize("over,err,what", [
    ({"y": torch.zeros(N, dtype=torch.int64)}, TypeError, "y"),
    ({"mask": torch.ones(N - 1, dtype=torch.uint8)}, ValueError, "mask"),
    ({"adv": torch.zeros(B, dtype=torch.float64)}, TypeError, "adv"),
    ({"ref_lp": torch.zeros(N + 3)}, ValueError, "ref_lp"),
    ({"H": torch.zeros(N + 1, d, dtype=torch.bfloat16)}, ValueError, "B \\* L"),
    ({"H": torch.zeros(N, d, dtype=torch.float16)}, TypeError, "float16"),
])
def test_forward_rejects_bad_arguments(over, err, what):
    with pytest.raises(err, match=what):
        _fwd(**over)


def test_reference_and_advantages_reject_bad_outputs():
    a = _args()
    with pytest.raises(ValueError, match="out"):
        gp.grpo_ref_logprobs(a["H"], a["W"], a["y"], out=torch.zeros(N - 1))
    with pytest.raises(TypeError, match="out"):
        gp.grpo_ref_logprobs(a["H"], a["W"], a["y"], out=torch.zeros(N, dtype=torch.float64))
    with pytest.raises(ValueError, match="y"):
        gp.grpo_ref_logprobs(a["H"], a["W"], torch.zeros(N + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        gp.grpo_advantages(torch.zeros(8), 4, out=torch.zeros(7))
    with pytest.raises(ValueError, match="group_size"):
        gp.grpo_advantages(torch.zeros(8), 3)


def test_fp8_calls_reject_bad_arguments():
    codes = torch.zeros(N, d, dtype=torch.uint8)
    Hq = gp.Fp8(codes, torch.ones(N), True)
    Wq = gp.Fp8(torch.zeros(V, d, dtype=torch.uint8), torch.ones(1), False)
    a = _args()
    with pytest.raises(ValueError, match="dH"):
        gp.grpo_loss_bwd_fp8(Hq, Wq, a["y"], a["mask"], a["adv"], a["ref_lp"], a["lp"], a["lse"],
                             B, L, dH=torch.zeros(N, d + 16, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="dH"):
        gp.grpo_loss_bwd_fp8(Hq, Wq, a["y"], a["mask"], a["adv"], a["ref_lp"], a["lp"], a["lse"],
                             B, L, dH=torch.zeros(N, d, dtype=torch.float32))
    with pytest.raises(ValueError, match="dW"):
        gp.grpo_loss_bwd_fp8(Hq, Wq, a["y"], a["mask"], a["adv"], a["ref_lp"], a["lp"], a["lse"],
                             B, L, dW=torch.zeros(V - 1, d))
    with pytest.raises(ValueError, match="H scales"):
        gp.grpo_loss_fwd_fp8(gp.Fp8(codes, torch.ones(N - 1), True), Wq, a["y"], a["mask"],
                             a["adv"], a["ref_lp"], B, L)
    with pytest.raises(ValueError, match="W codes"):
        gp.grpo_ref_logprobs_fp8(Hq, gp.Fp8(torch.zeros(V, d + 16, dtype=torch.uint8),
                                            torch.ones(1), False), a["y"])


def test_workspace_must_be_bytes():
    a = _args()
    with pytest.raises(TypeError, match="workspace"):
        gp.grpo_loss_fwd(a["H"], a["W"], a["y"], a["mask"], a["adv"], a["ref_lp"], B, L,
                         workspace=torch.zeros(1 << 20, dtype=torch.float32))
    with pytest.raises(ValueError, match="workspace"):
        gp.grpo_loss_fwd(a["H"], a["W"], a["y"], a["mask"], a["adv"], a["ref_lp"], B, L,
                         workspace=torch.zeros(16, dtype=torch.uint8))
