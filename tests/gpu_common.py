"""Shared helpers of the GPU parity tests: run the HIP chain (advantages ->
reference log-probs -> loss forward -> loss backward) through the C ABI, and
the float64 oracle chain on the very same inputs.  The two share nothing but
the seeded inputs; the oracle never sees a GPU output."""
import numpy as np
import torch

import oracle
import workloads
import grpo_policy_loss_amd as gp

BETA = workloads.BETA
EPS = workloads.EPS


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def bwd_workspace_for_slab(w, cols, chunk=None):
    """A backward workspace (uint8, on the GPU) sized for a dZ slab of `cols`
    vocabulary columns (a multiple of 256): the library plans its slab from the
    workspace size it is given."""
    chunk = w.chunk if chunk is None else chunk
    dt = gp.GRPO_F32 if w.dtype == "f32" else gp.GRPO_BF16
    cpad = -(-min(chunk, w.N) // 256) * 256
    es = 4 if w.dtype == "f32" else 2
    least = gp.grpo_workspace_bytes(gp.GRPO_OP_BWD_MIN, w.N, w.d, w.V, dt, chunk)
    return torch.empty(least + (cols - 256) * cpad * es, dtype=torch.uint8, device="cuda")


def gpu_chain(inp, w, beta=BETA, chunk=None, grad_loss=1.0, ref_from=None, opts=None,
              ws_bwd=None):
    """All outputs of the HIP path for inputs `inp` (tensors on the GPU).  ws_bwd:
    the backward's workspace (None: the default size)."""
    chunk = w.chunk if chunk is None else chunk
    adv = gp.grpo_advantages(inp["rewards"], w.G, EPS)
    H_ref = inp["H_ref"] if ref_from is None else ref_from
    ref = gp.grpo_ref_logprobs(H_ref, inp["W"], inp["y"], chunk, opts=opts)
    loss, lp, kl, lse = gp.grpo_loss_fwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref,
                                         w.B, w.L, beta, chunk, opts=opts)
    dH, dW = gp.grpo_loss_bwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref, lp, lse,
                              w.B, w.L, beta, grad_loss, chunk, opts=opts, workspace=ws_bwd)
    torch.cuda.synchronize()
    return dict(adv=adv, ref=ref, loss=loss, lp=lp, kl=kl, lse=lse, dH=dH, dW=dW)


def oracle_chain(inp, w, beta=BETA, grad_loss=1.0, backward=True, ref_from=None, opts=None):
    """Float64 oracle outputs for the same inputs (copied to the host)."""
    H, W = to64(inp["H"]), to64(inp["W"])
    H_ref = to64(inp["H_ref"] if ref_from is None else ref_from)
    y = inp["y"].cpu().numpy().astype(np.int64)
    mask = inp["mask"].cpu().numpy()
    adv = oracle.group_advantages(inp["rewards"].cpu().numpy(), w.G, EPS)
    ref, _ = oracle.token_logprobs(H_ref, W, y, opts=opts)
    out = oracle.loss_forward(H, W, y, mask, adv, ref, w.L, beta, opts=opts)
    out.update(adv=adv, ref=ref)
    if backward:
        dH, dW = oracle.loss_backward(H, W, y, mask, adv, ref, w.L, beta, grad_loss, opts=opts)
        out.update(dH=dH, dW=dW)
    return out


def cosine(a, b):
    a, b = np.ravel(a), np.ravel(b)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def max_abs_rel(got, want):
    """max |got - want| / max |want| over the tensor."""
    return float(np.abs(got - want).max() / max(np.abs(want).max(), 1e-300))
