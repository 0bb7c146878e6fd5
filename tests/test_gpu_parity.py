"""GPU parity of the HIP path against the float64 oracle, element by element,
at sizes that span several 256-wide tiles with ragged tails in tokens,
vocabulary and hidden size; plus the method's invariants on the GPU.

Tolerances.  float32 inputs: relative 1e-5 on the loss and on every lp.
bfloat16 inputs: relative 2e-3 on the loss, gradient cosine >= 0.999 and
max|g - g*| / max|g*| <= 1e-2 per tensor; lp within 1e-4 absolute (bf16
products are exact in fp32, so lp differs only by fp32 accumulation order)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import (BETA, bwd_workspace_for_slab, cosine, gpu_chain, max_abs_rel,
                              oracle_chain, to64)

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("grpo_policy_loss_amd")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


BASE = workloads.WORKLOADS[0]


def small(dtype, **kw):
    # 6 sequences x 100 tokens = 600 tokens (3 token tiles, last ragged), d = 320
    # (5 K slices of 64 bf16 / 10 of 32 f32), V = 1000 (4 vocab tiles, last 232 rows)
    args = dict(name="small", prompts=2, G=3, L=100, d=320, V=1000, dtype=dtype, chunk=256,
                len_lo=30, len_hi=100)
    args.update(kw)
    return BASE.scaled(**args)


def inputs(w, seed=0):
    return workloads.generate(w, seed=seed, device="cuda")


# ----------------------------------------------------------------------------- tile main loop
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (300, 517, 192), (1000, 77, 320), (33, 600, 8),
                                   (300, 517, 200)])
def test_tile_gemm_matches_exact_product(dtype, M, N, K):
    _need_gpu()
    if dtype == torch.float32 and K % 4:
        pytest.skip("f32 rows must be 16-byte multiples")
    g = torch.Generator(device="cuda").manual_seed(M * 7 + N * 3 + K)
    A = torch.randn(M, K, device="cuda", generator=g).to(dtype)
    B = torch.randn(N, K, device="cuda", generator=g).to(dtype)
    C = gp.grpo_gemm_nt(A, B)
    torch.cuda.synchronize()
    want = to64(A) @ to64(B).T
    err = np.abs(to64(C) - want).max()
    assert err <= 1e-5 * np.abs(want).max() + 1e-5, err


# K = 32 .. 832 bf16 elements: 1 to 13 slices of 128 bytes, whole or ending in a
# half slice, so the main loop ends in every phase of its three A slots and two B
# slots, with and without a k tail; M and N ragged.
@pytest.mark.parametrize("K", [32, 64, 96, 160, 192, 224, 288, 352, 416, 480, 544, 608, 704, 832])
def test_tile_gemm_every_slot_phase_and_k_tail(K):
    _need_gpu()
    g = torch.Generator(device="cuda").manual_seed(1000 + K)
    A = torch.randn(300, K, device="cuda", generator=g).to(torch.bfloat16)
    B = torch.randn(270, K, device="cuda", generator=g).to(torch.bfloat16)
    C = gp.grpo_gemm_nt(A, B)
    torch.cuda.synchronize()
    want = to64(A) @ to64(B).T
    err = np.abs(to64(C) - want).max()
    assert err <= 1e-5 * np.abs(want).max() + 1e-5, (K, err)


# ----------------------------------------------------------------------------- advantages
def test_advantages_match_oracle_and_degenerate_groups():
    _need_gpu()
    import oracle
    r = torch.tensor([0, 1, 2, 3, 3, 3, 3, 3, 1, 0, 2, 2], dtype=torch.float32, device="cuda")
    got = gp.grpo_advantages(r, 4, 1e-4).cpu().numpy()
    want = oracle.group_advantages(r.cpu().numpy(), 4, 1e-4)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)
    assert np.all(got[4:8] == 0.0)
    one = gp.grpo_advantages(r, 1, 1e-4).cpu().numpy()
    assert np.all(one == 0.0)
    big = torch.randint(0, 4, (3 * 100,), device="cuda").float()     # G > 64: strided lanes
    np.testing.assert_allclose(gp.grpo_advantages(big, 100).cpu().numpy(),
                               oracle.group_advantages(big.cpu().numpy(), 100, 1e-4),
                               rtol=1e-6, atol=1e-6)


# ----------------------------------------------------------------------------- full chain
@pytest.mark.parametrize("cols", [2048, 256])
def test_chain_bf16_multiple_vocab_slabs(cols):
    """bf16 path across slabs: a backward workspace with room for a slab of 2048
    (or the minimum 256) vocabulary columns splits V = 5000 into three or more
    slabs (the last one ragged), and the targets, uniform over V, fall in every
    slab."""
    _need_gpu()
    w = BASE.scaled(name="slabs-bf16", prompts=2, G=3, L=111, d=64, V=5000, dtype="bf16",
                    chunk=256, len_lo=50, len_hi=111)
    inp = inputs(w, seed=4)
    g = gpu_chain(inp, w, ws_bwd=bwd_workspace_for_slab(w, cols))
    o = oracle_chain(inp, w)
    assert abs(g["loss"].item() - o["loss"]) <= 2e-3 * abs(o["loss"])
    for k in ("dH", "dW"):
        assert cosine(to64(g[k]), o[k]) >= 0.999, k
        assert max_abs_rel(to64(g[k]), o[k]) <= 1e-2, k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [256, 300, 4096])
@pytest.mark.parametrize("d", [320, 200])
def test_chain_matches_oracle(dtype, chunk, d):
    # d = 200: the last K slice of every tile is partial (400 B of bf16 = 3 slices of
    # 128 B + 16 B; 800 B of f32 = 6 slices + 32 B), in the forward and the dZ recompute
    _need_gpu()
    w = small(dtype, chunk=chunk, d=d)
    inp = inputs(w, seed=1)
    g = gpu_chain(inp, w)
    o = oracle_chain(inp, w)
    lp, ref, lse, kl = to64(g["lp"]), to64(g["ref"]), to64(g["lse"]), to64(g["kl"])
    loss = float(g["loss"].item())
    np.testing.assert_allclose(to64(g["adv"]), o["adv"], rtol=1e-6, atol=1e-6)
    if dtype == "f32":
        np.testing.assert_allclose(lp, o["lp"], rtol=1e-5, atol=0)
        np.testing.assert_allclose(ref, o["ref"], rtol=1e-5, atol=0)
        np.testing.assert_allclose(lse, o["lse"], rtol=1e-5, atol=1e-6)
        assert abs(loss - o["loss"]) <= 1e-5 * abs(o["loss"])
        np.testing.assert_allclose(kl, o["kl"], rtol=1e-3, atol=1e-6)
        assert max_abs_rel(to64(g["dH"]), o["dH"]) <= 1e-4
        assert max_abs_rel(to64(g["dW"]), o["dW"]) <= 1e-4
    else:
        assert np.abs(lp - o["lp"]).max() <= 1e-4
        assert np.abs(ref - o["ref"]).max() <= 1e-4
        assert np.abs(lse - o["lse"]).max() <= 1e-4
        assert abs(loss - o["loss"]) <= 2e-3 * abs(o["loss"])
        assert np.abs(kl - o["kl"]).max() <= 1e-5
        for k in ("dH", "dW"):
            assert cosine(to64(g[k]), o[k]) >= 0.999, k
            assert max_abs_rel(to64(g[k]), o[k]) <= 1e-2, k
    # masked tokens get no gradient
    m = inp["mask"].cpu().numpy().astype(bool)
    assert np.all(to64(g["dH"])[~m] == 0.0)


def test_chain_multiple_vocab_slabs_and_chunks():
    """A backward workspace with room for 8192 vocabulary columns of a chunk of
    8192 f32 tokens splits V = 20000 into three or more slabs (the last one
    ragged); 8492 tokens need two chunks."""
    _need_gpu()
    w = BASE.scaled(name="slabs", prompts=1, G=4, L=2123, d=32, V=20000, dtype="f32",
                    chunk=8192, len_lo=1000, len_hi=2123)
    inp = inputs(w, seed=2)
    g = gpu_chain(inp, w, ws_bwd=bwd_workspace_for_slab(w, 8192))
    o = oracle_chain(inp, w)
    np.testing.assert_allclose(to64(g["lp"]), o["lp"], rtol=1e-5, atol=0)
    assert abs(g["loss"].item() - o["loss"]) <= 1e-5 * abs(o["loss"])
    assert max_abs_rel(to64(g["dH"]), o["dH"]) <= 1e-4
    assert max_abs_rel(to64(g["dW"]), o["dW"]) <= 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_policy_equals_reference_kl_is_exactly_zero(dtype):
    _need_gpu()
    w = small(dtype)
    inp = inputs(w, seed=3)
    g = gpu_chain(inp, w, ref_from=inp["H"])
    assert torch.equal(g["ref"], g["lp"])
    assert torch.all(g["kl"] == 0)
    A = np.repeat(g["adv"].cpu().numpy().astype(np.float64), w.L)
    m = inp["mask"].cpu().numpy().astype(np.float64)
    assert abs(g["loss"].item() - (-(m * A).sum() / m.sum())) <= 1e-6


def test_bitwise_determinism_and_chunk_invariance():
    _need_gpu()
    w = small("bf16")
    inp = inputs(w, seed=4)
    a = gpu_chain(inp, w, chunk=256)
    b = gpu_chain(inp, w, chunk=256)
    for k in ("loss", "lp", "kl", "lse", "ref", "dH", "dW"):
        assert torch.equal(a[k], b[k]), k
    c = gpu_chain(inp, w, chunk=512)
    assert torch.equal(a["lp"], c["lp"]) and torch.equal(a["lse"], c["lse"])


def test_empty_mask_gives_zero_loss_and_gradients():
    _need_gpu()
    w = small("f32")
    inp = inputs(w, seed=5)
    inp["mask"].zero_()
    g = gpu_chain(inp, w)
    assert g["loss"].item() == 0.0
    assert torch.all(g["dH"] == 0) and torch.all(g["dW"] == 0)


def test_dw_accumulates_and_grad_loss_scales():
    _need_gpu()
    w = small("f32")
    inp = inputs(w, seed=6)
    g = gpu_chain(inp, w)
    dH2, dW2 = gp.grpo_loss_bwd(inp["H"], inp["W"], inp["y"], inp["mask"], g["adv"], g["ref"],
                                g["lp"], g["lse"], w.B, w.L, BETA, -2.0, w.chunk,
                                dW=g["dW"].clone())
    torch.cuda.synchronize()
    np.testing.assert_allclose(to64(dW2), -1.0 * to64(g["dW"]), rtol=1e-5,
                               atol=1e-6 * np.abs(to64(g["dW"])).max())
    np.testing.assert_allclose(to64(dH2), -2.0 * to64(g["dH"]), rtol=1e-5,
                               atol=1e-6 * np.abs(to64(g["dH"])).max())


@pytest.mark.parametrize("N,d,V", [(1, 8, 1), (7, 16, 3), (257, 8, 300)])
def test_degenerate_shapes_pure_kl(N, d, V):
    """One sequence (G = 1, so every advantage is 0): the gradient is the KL
    term alone.  The reference hidden states are drawn independently, so
    x = ref_lp - lp is O(1) and the KL gradient is well conditioned in fp32
    (with H_ref = H + small noise, x is a difference of two nearly equal fp32
    log-probs and carries ~1e-4 relative error by construction)."""
    _need_gpu()
    w = BASE.scaled(name="tiny", prompts=1, G=1, L=N, d=d, V=V, dtype="f32", chunk=100,
                    len_lo=max(1, N // 2), len_hi=N)
    inp = inputs(w, seed=7)
    ref_h = workloads.draw_hidden(N, d, torch.float32, 99, "cuda")
    g = gpu_chain(inp, w, ref_from=ref_h)
    o = oracle_chain(inp, w, ref_from=ref_h)
    assert np.all(o["adv"] == 0)
    np.testing.assert_allclose(to64(g["lp"]), o["lp"], rtol=1e-5, atol=1e-6)
    assert abs(g["loss"].item() - o["loss"]) <= 1e-5 * abs(o["loss"]) + 1e-7
    if V == 1:          # a single class: lp = 0, no gradient at all
        assert torch.all(g["dW"] == 0) and torch.all(g["dH"] == 0)
    else:
        assert max_abs_rel(to64(g["dW"]), o["dW"]) <= 1e-4
        assert max_abs_rel(to64(g["dH"]), o["dH"]) <= 1e-4


XFORMS = [
    {"temperature": 0.7},
    {"logit_softcapping": 3.0},
    {"logit_scale_multiply": 1.3, "logit_scale_divide": 0.8, "logit_softcapping": 2.5,
     "temperature": 1.25},
]


@pytest.mark.parametrize("opts", XFORMS, ids=["temperature", "softcap", "all"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_with_logit_transform_matches_oracle(dtype, opts):
    """Scale, softcap and temperature through the whole chain (ragged V = 1000,
    chunks of 256 over 600 tokens) against the oracle's transformed logits."""
    _need_gpu()
    w = small(dtype)
    inp = inputs(w, seed=8)
    g = gpu_chain(inp, w, opts=opts)
    o = oracle_chain(inp, w, opts=opts)
    if dtype == "f32":
        np.testing.assert_allclose(to64(g["ref"]), o["ref"], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(to64(g["lp"]), o["lp"], rtol=1e-5, atol=1e-6)
        assert abs(g["loss"].item() - o["loss"]) <= 1e-5 * abs(o["loss"])
        for k in ("dH", "dW"):
            assert max_abs_rel(to64(g[k]), o[k]) <= 1e-4, k
    else:
        assert np.abs(to64(g["lp"]) - o["lp"]).max() <= 1e-4
        assert abs(g["loss"].item() - o["loss"]) <= 2e-3 * abs(o["loss"])
        for k in ("dH", "dW"):
            assert cosine(to64(g[k]), o[k]) >= 0.999, k
            assert max_abs_rel(to64(g[k]), o[k]) <= 1e-2, k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_logit_transform_keeps_kl_exactly_zero_for_policy_equal_reference(dtype):
    _need_gpu()
    w = small(dtype)
    inp = inputs(w, seed=9)
    g = gpu_chain(inp, w, ref_from=inp["H"], opts=XFORMS[2])
    assert torch.equal(g["ref"], g["lp"])
    assert torch.all(g["kl"] == 0)


VARIANTS = [
    {"kl_estimator": 1},
    {"kl_estimator": 2},
    {"no_detach": 1},
    {"aggregation": 1},
    {"kl_estimator": 1, "no_detach": 1, "aggregation": 1, "temperature": 0.9},
]
VARIANT_IDS = ["forward-kl", "reverse-kl-q", "no-detach", "sequence-mean", "combined"]


@pytest.mark.parametrize("opts", VARIANTS, ids=VARIANT_IDS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_with_loss_variant_matches_oracle(dtype, opts):
    """The ablation's estimator, detach and aggregation variants through the
    whole chain (ragged tiles, 3 chunks); sequence 2 has an empty mask, so the
    per-sequence mean counts it in B with a zero contribution.  The reference
    hidden states are drawn independently, as in the pure-KL test above: x =
    ref_lp - lp is then O(1), so the KL terms (all of the no-detach gradient)
    are well conditioned in fp32 and every estimator is exercised away from 0."""
    _need_gpu()
    w = small(dtype)
    inp = inputs(w, seed=10)
    inp["mask"][2 * w.L:3 * w.L] = 0
    ref_h = workloads.draw_hidden(w.N, w.d, inp["H"].dtype, 98, "cuda")
    g = gpu_chain(inp, w, ref_from=ref_h, opts=opts)
    o = oracle_chain(inp, w, ref_from=ref_h, opts=opts)
    print(f"[variant] {dtype} {opts} loss gpu {g['loss'].item():.7g} oracle {o['loss']:.7g}",
          flush=True)
    # the kernel's estimator arithmetic (fp32) against the same estimator in float64
    # on the GPU's own lp and ref; lp itself is checked against the oracle below
    np.testing.assert_allclose(to64(g["kl"]), oracle.token_kl(to64(g["ref"]), to64(g["lp"]), opts),
                               rtol=1e-5, atol=1e-7)
    if dtype == "f32":
        np.testing.assert_allclose(to64(g["lp"]), o["lp"], rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(to64(g["kl"]), o["kl"], rtol=1e-3, atol=1e-6)
        assert abs(g["loss"].item() - o["loss"]) <= 1e-5 * abs(o["loss"])
        for k in ("dH", "dW"):
            assert max_abs_rel(to64(g[k]), o[k]) <= 1e-4, k
    else:
        assert np.abs(to64(g["lp"]) - o["lp"]).max() <= 1e-4
        assert abs(g["loss"].item() - o["loss"]) <= 2e-3 * abs(o["loss"])
        for k in ("dH", "dW"):
            assert cosine(to64(g[k]), o[k]) >= 0.999, k
            assert max_abs_rel(to64(g[k]), o[k]) <= 1e-2, k
    m = inp["mask"].cpu().numpy().astype(bool)
    assert np.all(to64(g["dH"])[~m] == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_detach_gradient_is_bitwise_the_zero_advantage_gradient(dtype):
    """Without the detach the advantage term has no gradient: the backward equals,
    bit for bit, the detached backward with every advantage zero."""
    _need_gpu()
    w = small(dtype)
    inp = inputs(w, seed=11)
    g = gpu_chain(inp, w, opts={"no_detach": 1})
    adv0 = torch.zeros_like(g["adv"])
    dH0, dW0 = gp.grpo_loss_bwd(inp["H"], inp["W"], inp["y"], inp["mask"], adv0, g["ref"],
                                g["lp"], g["lse"], w.B, w.L, BETA, 1.0, w.chunk)
    torch.cuda.synchronize()
    assert torch.equal(g["dH"], dH0)
    assert torch.equal(g["dW"], dW0)


@pytest.mark.parametrize("kl_estimator", [0, 1, 2])
def test_sequence_mean_policy_equals_reference_gives_zero_loss(kl_estimator):
    """With kl = 0 the per-sequence mean is -mean_b(A_b), zero up to the rounding
    of the group advantages; the token mean of the same inputs is not."""
    _need_gpu()
    w = small("f32")
    inp = inputs(w, seed=12)
    g = gpu_chain(inp, w, ref_from=inp["H"], opts={"kl_estimator": kl_estimator, "aggregation": 1})
    t = gpu_chain(inp, w, ref_from=inp["H"], opts={"kl_estimator": kl_estimator})
    assert torch.all(g["kl"] == 0)
    assert abs(g["loss"].item()) <= 1e-6
    assert abs(t["loss"].item()) > 1e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_with_automatic_chunk_matches_fixed_chunk_bitwise(dtype):
    """chunk = 0 resolves through grpo_auto_chunk (half the free HBM); lp and lse
    do not depend on the chunk, so they equal a fixed-chunk run bit for bit, and
    the whole chain still matches the oracle."""
    _need_gpu()
    w = small(dtype)
    inp = inputs(w, seed=13)
    a = gpu_chain(inp, w, chunk=0)
    f = gpu_chain(inp, w, chunk=256)
    assert torch.equal(a["lp"], f["lp"]) and torch.equal(a["lse"], f["lse"])
    assert torch.equal(a["ref"], f["ref"])
    o = oracle_chain(inp, w)
    tol = 1e-5 if dtype == "f32" else 2e-3
    assert abs(a["loss"].item() - o["loss"]) <= tol * abs(o["loss"])
    for k in ("dH", "dW"):
        assert cosine(to64(a[k]), o[k]) >= 0.999, k
