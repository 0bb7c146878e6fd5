"""Full-size GPU parity: every benchmark workload at its real shape, in the
launch configuration the benchmark times (same chunk), checked against the
float64 oracle on outputs the oracle can compute one by one:

  * lp, ref_lp, lse and kl of 256 sampled tokens (full logits row each);
  * dH rows of 256 sampled unmasked tokens (needs only those rows' logits,
    the global unmasked count and the advantages);
  * dW in full from a second backward at the same shape whose mask keeps a
    sparse set of tokens spread over every chunk (dW is then an exact sum
    the oracle forms from those rows' logits);
  * properties that hold at any size for the dense run: the loss equals the
    masked mean of the per-token terms -(A - beta kl), the KL is >= 0, the
    vocabulary-sum of dW vanishes and masked tokens get no dH.

Tolerances (bf16 inputs, fp32 accumulation): lp/ref/lse within 2e-4
absolute, kl within 1e-5 absolute; gradient cosine >= 0.999 and
max|g - g*| / max|g*| <= 1e-2."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import BETA, EPS, cosine, max_abs_rel, to64

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("grpo_policy_loss_amd")

FULL = [w.name for w in workloads.WORKLOADS[1:]]


def _sample_rows(N, L, n, rng, extra=()):
    rows = set(int(x) for x in rng.choice(N, size=n, replace=False))
    rows.update(int(x) for x in extra if 0 <= x < N)
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = workloads.BY_NAME[name]
    print(f"[full] {name}: N={w.N} d={w.d} V={w.V} chunk={w.chunk}", flush=True)
    inp = workloads.generate(w, seed=11, device="cuda")
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    adv = gp.grpo_advantages(inp["rewards"], w.G, EPS)
    ref = gp.grpo_ref_logprobs(inp["H_ref"], inp["W"], inp["y"], w.chunk)
    loss, lp, kl, lse = gp.grpo_loss_fwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref,
                                         w.B, w.L, BETA, w.chunk)
    dH, dW = gp.grpo_loss_bwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref, lp, lse,
                              w.B, w.L, BETA, 1.0, w.chunk)
    torch.cuda.synchronize()
    # everything the calls allocate (workspaces, dH, dW and the per-token outputs) stays
    # below one bf16 tokens x vocab tensor: no (tokens x vocab) tensor is ever resident
    extra = torch.cuda.max_memory_allocated() - base
    print(f"[full] {name}: peak allocated by the calls {extra / 1e9:.2f} GB against "
          f"N x V x 2 B = {w.N * w.V * 2 / 1e9:.2f} GB", flush=True)
    assert extra < w.N * w.V * 2

    mask = inp["mask"].cpu().numpy()
    y = inp["y"].cpu().numpy().astype(np.int64)
    A = oracle.group_advantages(inp["rewards"].cpu().numpy(), w.G, EPS)
    np.testing.assert_allclose(adv.cpu().numpy(), A, rtol=1e-6, atol=1e-6)
    W64 = to64(inp["W"])
    rng = np.random.default_rng(5)
    # samples include chunk boundaries and the very last token
    edges = [0, w.N - 1] + [c * w.chunk + o for c in range(1, w.N // w.chunk) for o in (-1, 0)]
    rows = _sample_rows(w.N, w.L, 256, rng, edges)
    H_rows = to64(inp["H"][torch.as_tensor(rows, device="cuda")])
    R_rows = to64(inp["H_ref"][torch.as_tensor(rows, device="cuda")])
    o_lp, o_lse = oracle.token_logprobs(H_rows, W64, y[rows])
    o_ref, _ = oracle.token_logprobs(R_rows, W64, y[rows])
    o_kl = oracle.reverse_kl_k3(o_ref, o_lp)
    g_lp, g_ref, g_lse, g_kl = (to64(t)[rows] for t in (lp, ref, lse, kl))
    print(f"[full] {name}: max|dlp| {np.abs(g_lp - o_lp).max():.2e} "
          f"max|dlse| {np.abs(g_lse - o_lse).max():.2e} max|dkl| {np.abs(g_kl - o_kl).max():.2e}",
          flush=True)
    assert np.abs(g_lp - o_lp).max() <= 2e-4
    assert np.abs(g_ref - o_ref).max() <= 2e-4
    assert np.abs(g_lse - o_lse).max() <= 2e-4
    assert np.abs(g_kl - o_kl).max() <= 1e-5

    # loss: masked mean of -(A - beta kl), with A the oracle's and kl the GPU's (checked above)
    m = mask.astype(np.float64)
    A_t = np.repeat(A, w.L)
    kl_all = to64(kl)
    assert np.all(kl_all >= 0)
    want_loss = float((m * -(A_t - BETA * kl_all)).sum() / m.sum())
    assert abs(loss.item() - want_loss) <= 2e-3 * abs(want_loss)

    # dH on sampled unmasked rows, oracle from those rows' own logits
    act = np.nonzero(mask)[0]
    drows = np.array(sorted(set(rng.choice(act, size=min(256, len(act)), replace=False).tolist())))
    H64 = np.zeros((w.N, w.d))        # only the requested rows are read by the oracle
    H64[drows] = to64(inp["H"][torch.as_tensor(drows, device="cuda")])
    ref64 = np.zeros(w.N)
    Rd = to64(inp["H_ref"][torch.as_tensor(drows, device="cuda")])
    ref64[drows], _ = oracle.token_logprobs(Rd, W64, y[drows])
    o_dH, _ = oracle.loss_backward(H64, W64, y, mask, A, ref64, w.L, BETA, dh_rows=drows,
                                   want_dW=False)
    g_dH = to64(dH[torch.as_tensor(drows, device="cuda")])
    print(f"[full] {name}: dH rows cos {cosine(g_dH, o_dH):.6f} "
          f"maxrel {max_abs_rel(g_dH, o_dH):.2e}", flush=True)
    assert cosine(g_dH, o_dH) >= 0.999
    assert max_abs_rel(g_dH, o_dH) <= 1e-2
    masked = np.nonzero(mask == 0)[0]
    if len(masked):
        assert torch.all(dH[torch.as_tensor(masked[:4096], device="cuda")] == 0)
    # dW of the dense run: each dZ row sums to zero, so sum_v dW[v, :] vanishes up to the
    # bf16 rounding of dZ (about 2^-9 |c_t| per token); a sign or index slip gives ratio ~1
    Wd = dW.double()
    ratio = (Wd.sum(dim=0).abs() / Wd.abs().sum(dim=0).clamp(min=1e-300)).max().item()
    print(f"[full] {name}: max_k |sum_v dW| / sum_v |dW| = {ratio:.2e}", flush=True)
    assert ratio <= 1e-2


@pytest.mark.parametrize("name", FULL)
def test_full_size_exact_dW_with_sparse_mask(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = workloads.BY_NAME[name]
    print(f"[full-dW] {name}", flush=True)
    inp = workloads.generate(w, seed=12, device="cuda")
    rng = np.random.default_rng(7)
    keep = set(int(x) for x in rng.choice(w.N, size=64, replace=False))
    keep.update(c * w.chunk for c in range(w.N // w.chunk))      # one at every chunk start
    keep.add(w.N - 1)
    keep = np.array(sorted(keep))
    mask = torch.zeros(w.N, dtype=torch.uint8, device="cuda")
    mask[torch.as_tensor(keep, device="cuda")] = 1
    adv = gp.grpo_advantages(inp["rewards"], w.G, EPS)
    ref = gp.grpo_ref_logprobs(inp["H_ref"], inp["W"], inp["y"], w.chunk)
    loss, lp, kl, lse = gp.grpo_loss_fwd(inp["H"], inp["W"], inp["y"], mask, adv, ref, w.B, w.L,
                                         BETA, w.chunk)
    dH, dW = gp.grpo_loss_bwd(inp["H"], inp["W"], inp["y"], mask, adv, ref, lp, lse, w.B, w.L,
                              BETA, 1.0, w.chunk)
    torch.cuda.synchronize()

    y = inp["y"].cpu().numpy().astype(np.int64)
    A = oracle.group_advantages(inp["rewards"].cpu().numpy(), w.G, EPS)
    W64 = to64(inp["W"])
    H64 = np.zeros((w.N, w.d))
    H64[keep] = to64(inp["H"][torch.as_tensor(keep, device="cuda")])
    ref64 = np.zeros(w.N)
    ref64[keep], _ = oracle.token_logprobs(to64(inp["H_ref"][torch.as_tensor(keep, device="cuda")]),
                                           W64, y[keep])
    o_dH, o_dW = oracle.loss_backward(H64, W64, y, mask.cpu().numpy(), A, ref64, w.L, BETA,
                                      dh_rows=keep)
    g_dW = to64(dW)
    print(f"[full-dW] {name}: dW cos {cosine(g_dW, o_dW):.6f} maxrel {max_abs_rel(g_dW, o_dW):.2e}",
          flush=True)
    assert cosine(g_dW, o_dW) >= 0.999
    assert max_abs_rel(g_dW, o_dW) <= 1e-2
    g_dH = to64(dH[torch.as_tensor(keep, device="cuda")])
    assert cosine(g_dH, o_dH) >= 0.999
    assert max_abs_rel(g_dH, o_dH) <= 1e-2
    # every other row of dH is zero
    others = torch.ones(w.N, dtype=torch.bool, device="cuda")
    others[torch.as_tensor(keep, device="cuda")] = False
    assert torch.all(dH[others] == 0)


@pytest.mark.parametrize("opts", [
    {"logit_softcapping": 30.0, "temperature": 0.9},
    {"logit_softcapping": 30.0, "temperature": 0.9, "kl_estimator": 1, "aggregation": 1}],
    ids=["transform", "transform+forward-kl+sequence-mean"])
def test_full_size_logit_transform_sampled_parity(opts):
    """Qwen2.5-1.5B shape with softcap 30 and temperature 0.9 (the launch
    configuration the benchmark times, plus the transform), also with the forward
    KL and the per-sequence mean: lp/ref/lse/kl of sampled tokens and dH of
    sampled active rows against the oracle's transformed logits."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = workloads.BY_NAME["qwen2.5-1.5b-bf16"]
    print(f"[full-xform] {w.name} {opts}", flush=True)
    inp = workloads.generate(w, seed=13, device="cuda")
    adv = gp.grpo_advantages(inp["rewards"], w.G, EPS)
    ref = gp.grpo_ref_logprobs(inp["H_ref"], inp["W"], inp["y"], w.chunk, opts=opts)
    loss, lp, kl, lse = gp.grpo_loss_fwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref,
                                         w.B, w.L, BETA, w.chunk, opts=opts)
    dH, dW = gp.grpo_loss_bwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv, ref, lp, lse,
                              w.B, w.L, BETA, 1.0, w.chunk, opts=opts)
    torch.cuda.synchronize()
    y = inp["y"].cpu().numpy().astype(np.int64)
    mask = inp["mask"].cpu().numpy()
    A = oracle.group_advantages(inp["rewards"].cpu().numpy(), w.G, EPS)
    W64 = to64(inp["W"])
    rng = np.random.default_rng(17)
    rows = _sample_rows(w.N, w.L, 256, rng, [0, w.N - 1])
    o_lp, o_lse = oracle.token_logprobs(to64(inp["H"][torch.as_tensor(rows, device="cuda")]), W64,
                                        y[rows], opts=opts)
    o_ref, _ = oracle.token_logprobs(to64(inp["H_ref"][torch.as_tensor(rows, device="cuda")]), W64,
                                     y[rows], opts=opts)
    g_lp, g_ref, g_lse = (to64(t)[rows] for t in (lp, ref, lse))
    print(f"[full-xform] max|dlp| {np.abs(g_lp - o_lp).max():.2e} "
          f"max|dlse| {np.abs(g_lse - o_lse).max():.2e}", flush=True)
    assert np.abs(g_lp - o_lp).max() <= 2e-4
    assert np.abs(g_ref - o_ref).max() <= 2e-4
    assert np.abs(g_lse - o_lse).max() <= 2e-4
    # the GPU's kl against the estimator evaluated in float64 on its own lp and ref
    g_kl = to64(kl)[rows]
    np.testing.assert_allclose(g_kl, oracle.token_kl(g_ref, g_lp, opts), rtol=1e-4, atol=1e-6)
    act = np.nonzero(mask)[0]
    drows = np.array(sorted(set(rng.choice(act, size=256, replace=False).tolist())))
    H64 = np.zeros((w.N, w.d))
    H64[drows] = to64(inp["H"][torch.as_tensor(drows, device="cuda")])
    ref64 = np.zeros(w.N)
    ref64[drows], _ = oracle.token_logprobs(to64(inp["H_ref"][torch.as_tensor(drows, device="cuda")]),
                                            W64, y[drows], opts=opts)
    o_dH, _ = oracle.loss_backward(H64, W64, y, mask, A, ref64, w.L, BETA, dh_rows=drows,
                                   want_dW=False, opts=opts)
    g_dH = to64(dH[torch.as_tensor(drows, device="cuda")])
    print(f"[full-xform] dH rows cos {cosine(g_dH, o_dH):.6f} maxrel {max_abs_rel(g_dH, o_dH):.2e}",
          flush=True)
    assert cosine(g_dH, o_dH) >= 0.999
    assert max_abs_rel(g_dH, o_dH) <= 1e-2
