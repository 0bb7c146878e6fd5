"""GPU parity of the fp8 (e4m3) path: the quantizer bit for bit against the
oracle's (codes and scales decide integers, so both sides take them exactly),
and the fp8 loss chain against the float64 oracle evaluated on the oracle's
own dequantised inputs.

Tolerances: e4m3 x e4m3 products are exact in float32 and the scales are
powers of two, so the GPU logits differ from the float64 ones only by float32
accumulation; the bf16 bounds apply (|dlp| <= 1e-4, loss relative 2e-3,
gradient cosine >= 0.999 and max-abs-rel <= 1e-2; the backward recomputes
logits through the bfloat16 loop on exact copies, so its logits differ from
the forward's only in summation order)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_common import BETA, EPS, cosine, max_abs_rel, to64

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("grpo_policy_loss_amd")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


BASE = workloads.WORKLOADS[0]


def small(**kw):
    args = dict(name="small-fp8", prompts=2, G=3, L=100, d=320, V=1000, dtype="bf16", chunk=256,
                len_lo=30, len_hi=100)
    args.update(kw)
    return BASE.scaled(**args)


def _special_rows(cols):
    """Rows whose largest magnitude is 448 (scale 1), holding exact values and
    midpoints between e4m3 neighbours (ties to even), subnormals and zeros."""
    vals = [448.0, 1.0625, 1.1875, -1.0625, 432.0, 400.0, 416.0, 0.0029296875,
            0.0068359375, 0.0146484375, 0.001953125, -0.0, 0.0, 3.0, -5.5, 0.4375]
    r = np.zeros((3, cols))
    r[0, :len(vals)] = vals
    r[1] = 0.0                                        # all-zero row: scale 1, codes 0
    r[2, :len(vals)] = np.array(vals) * 2.0 ** -10    # the same pattern, scale 2^-10
    return r


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("per_row", [True, False])
def test_quantize_matches_oracle_bitwise(dtype, per_row):
    _need_gpu()
    g = torch.Generator(device="cuda").manual_seed(5)
    X = torch.randn(600, 320, device="cuda", generator=g) * torch.exp2(
        torch.randint(-8, 8, (600, 1), device="cuda", generator=g).float())
    X[:3] = torch.tensor(_special_rows(320), dtype=torch.float32, device="cuda")
    X = X.to(dtype).contiguous()
    print(f"[fp8-quant] {dtype} per_row={per_row}", flush=True)
    q = gp.quantize_fp8(X, per_row=per_row)
    torch.cuda.synchronize()
    codes, sc = oracle.fp8_quantize(to64(X), per_row=per_row)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), codes)
    np.testing.assert_array_equal(q.scales.cpu().double().numpy(), sc)
    # dequantisation is exact
    np.testing.assert_array_equal(to64(gp.dequantize_fp8(q)), oracle.fp8_dequantize(codes, sc))


def _fp8_inputs(w, seed, ref_equal=False):
    inp = workloads.generate(w, seed=seed, device="cuda")
    Hq = gp.quantize_fp8(inp["H"], per_row=True)
    Rq = Hq if ref_equal else gp.quantize_fp8(inp["H_ref"], per_row=True)
    Wq = gp.quantize_fp8(inp["W"], per_row=False)
    return inp, Hq, Rq, Wq


def _oracle_deq(X):
    """The oracle's own per-row quantisation of X, dequantised (float64)."""
    codes, sc = oracle.fp8_quantize(to64(X), per_row=True)
    return oracle.fp8_dequantize(codes, sc)


def _oracle_w(W, block=8192):
    """The oracle's per-tensor quantisation of W, dequantised: the tensor's
    exponent, then the e4m3 codes of each block of rows (fp8_quantize's steps,
    in row blocks to bound host memory at the full vocabulary)."""
    e = oracle.fp8_scale_exponent(float(W.abs().max().item()))
    out = np.empty(tuple(W.shape))
    for r0 in range(0, W.shape[0], block):
        Xb = to64(W[r0:r0 + block])
        out[r0:r0 + block] = oracle.fp8_e4m3_decode(oracle.fp8_e4m3_encode(Xb / 2.0 ** e)) * 2.0 ** e
    return out


def _gpu_chain_fp8(inp, w, Hq, Rq, Wq, chunk, opts=None):
    adv = gp.grpo_advantages(inp["rewards"], w.G, EPS)
    ref = gp.grpo_ref_logprobs_fp8(Rq, Wq, inp["y"], chunk, opts=opts)
    loss, lp, kl, lse = gp.grpo_loss_fwd_fp8(Hq, Wq, inp["y"], inp["mask"], adv, ref, w.B, w.L,
                                             BETA, chunk, opts=opts)
    dH, dW = gp.grpo_loss_bwd_fp8(Hq, Wq, inp["y"], inp["mask"], adv, ref, lp, lse, w.B, w.L,
                                  BETA, 1.0, chunk, opts=opts)
    torch.cuda.synchronize()
    return dict(adv=adv, ref=ref, loss=loss, lp=lp, kl=kl, lse=lse, dH=dH, dW=dW)


@pytest.mark.parametrize("chunk", [256, 4096])
@pytest.mark.parametrize("opts", [None, {"logit_softcapping": 3.0, "temperature": 0.8}],
                         ids=["plain", "softcap+temperature"])
def test_fp8_chain_matches_oracle_on_dequantised_inputs(chunk, opts):
    """600 tokens in chunks, d = 320 (2.5 fp8 slices: a K tail and an odd slice
    count), V = 1000 (ragged last vocabulary tile)."""
    _need_gpu()
    w = small(chunk=chunk)
    inp, Hq, Rq, Wq = _fp8_inputs(w, seed=21)
    print(f"[fp8-chain] chunk={chunk} opts={opts}", flush=True)
    g = _gpu_chain_fp8(inp, w, Hq, Rq, Wq, chunk, opts)
    H, R, W = _oracle_deq(inp["H"]), _oracle_deq(inp["H_ref"]), _oracle_w(inp["W"])
    y = inp["y"].cpu().numpy().astype(np.int64)
    mask = inp["mask"].cpu().numpy()
    A = oracle.group_advantages(inp["rewards"].cpu().numpy(), w.G, EPS)
    o_ref, _ = oracle.token_logprobs(R, W, y, opts=opts)
    o = oracle.loss_forward(H, W, y, mask, A, o_ref, w.L, BETA, opts=opts)
    o_dH, o_dW = oracle.loss_backward(H, W, y, mask, A, o_ref, w.L, BETA, 1.0, opts=opts)
    print(f"[fp8-chain] max|dlp| {np.abs(to64(g['lp']) - o['lp']).max():.2e} loss gpu "
          f"{g['loss'].item():.7g} oracle {o['loss']:.7g}", flush=True)
    assert np.abs(to64(g["ref"]) - o_ref).max() <= 1e-4
    assert np.abs(to64(g["lp"]) - o["lp"]).max() <= 1e-4
    assert np.abs(to64(g["lse"]) - o["lse"]).max() <= 1e-4
    assert abs(g["loss"].item() - o["loss"]) <= 2e-3 * abs(o["loss"])
    for k, ov in (("dH", o_dH), ("dW", o_dW)):
        assert cosine(to64(g[k]), ov) >= 0.999, k
        assert max_abs_rel(to64(g[k]), ov) <= 1e-2, k
    m = mask.astype(bool)
    assert np.all(to64(g["dH"])[~m] == 0.0)


def test_fp8_policy_equal_reference_gives_exactly_zero_kl():
    _need_gpu()
    w = small()
    inp, Hq, Rq, Wq = _fp8_inputs(w, seed=22, ref_equal=True)
    g = _gpu_chain_fp8(inp, w, Hq, Rq, Wq, w.chunk)
    assert torch.equal(g["ref"], g["lp"])
    assert torch.all(g["kl"] == 0)


def test_fp8_full_size_sampled_parity():
    """Qwen2.5-1.5B shape (32768 tokens, d 1536, V 151936, chunk 4096) through the
    fp8 forward: lp/ref/lse of 256 sampled tokens against the oracle on its own
    dequantised rows."""
    _need_gpu()
    w = workloads.BY_NAME["qwen2.5-1.5b-bf16"]
    print(f"[fp8-full] {w.name}", flush=True)
    inp, Hq, Rq, Wq = _fp8_inputs(w, seed=23)
    adv = gp.grpo_advantages(inp["rewards"], w.G, EPS)
    ref = gp.grpo_ref_logprobs_fp8(Rq, Wq, inp["y"], w.chunk)
    loss, lp, kl, lse = gp.grpo_loss_fwd_fp8(Hq, Wq, inp["y"], inp["mask"], adv, ref, w.B, w.L,
                                             BETA, w.chunk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(24)
    rows = np.unique(np.concatenate([rng.integers(0, w.N, 254), [0, w.N - 1]]))
    W = _oracle_w(inp["W"])
    idx = torch.as_tensor(rows, device="cuda")
    H = _oracle_deq(inp["H"][idx])
    R = _oracle_deq(inp["H_ref"][idx])
    y = inp["y"].cpu().numpy().astype(np.int64)[rows]
    o_lp, o_lse = oracle.token_logprobs(H, W, y)
    o_ref, _ = oracle.token_logprobs(R, W, y)
    g_lp, g_lse, g_ref = (to64(t)[rows] for t in (lp, lse, ref))
    print(f"[fp8-full] max|dlp| {np.abs(g_lp - o_lp).max():.2e} max|dlse| "
          f"{np.abs(g_lse - o_lse).max():.2e}", flush=True)
    assert np.abs(g_lp - o_lp).max() <= 2e-4
    assert np.abs(g_ref - o_ref).max() <= 2e-4
    assert np.abs(g_lse - o_lse).max() <= 2e-4
    np.testing.assert_allclose(to64(kl)[rows], oracle.token_kl(g_ref, g_lp), rtol=1e-4, atol=1e-6)


def test_fp8_full_size_backward_sampled_parity():
    """Qwen2.5-1.5B shape through the fp8 forward and backward, in the launch
    configuration `bench.py --fp8` times (chunk 4096): dH of 256 sampled active
    rows of the dense run, and dW in full from a second backward whose mask keeps
    a sparse set of tokens spread over every chunk, against the oracle on its own
    dequantised H, H_ref and W."""
    _need_gpu()
    w = workloads.BY_NAME["qwen2.5-1.5b-bf16"]
    print(f"[fp8-full-bwd] {w.name}", flush=True)
    inp, Hq, Rq, Wq = _fp8_inputs(w, seed=25)
    adv = gp.grpo_advantages(inp["rewards"], w.G, EPS)
    ref = gp.grpo_ref_logprobs_fp8(Rq, Wq, inp["y"], w.chunk)
    _, lp, _, lse = gp.grpo_loss_fwd_fp8(Hq, Wq, inp["y"], inp["mask"], adv, ref, w.B, w.L,
                                         BETA, w.chunk)
    dH, dW = gp.grpo_loss_bwd_fp8(Hq, Wq, inp["y"], inp["mask"], adv, ref, lp, lse, w.B, w.L,
                                  BETA, 1.0, w.chunk)
    rng = np.random.default_rng(26)
    keep = set(int(x) for x in rng.choice(w.N, size=64, replace=False))
    keep.update(c * w.chunk for c in range(w.N // w.chunk))
    keep.add(w.N - 1)
    keep = np.array(sorted(keep))
    smask = torch.zeros(w.N, dtype=torch.uint8, device="cuda")
    smask[torch.as_tensor(keep, device="cuda")] = 1
    _, lp_s, _, lse_s = gp.grpo_loss_fwd_fp8(Hq, Wq, inp["y"], smask, adv, ref, w.B, w.L, BETA,
                                             w.chunk)
    dH_s, dW_s = gp.grpo_loss_bwd_fp8(Hq, Wq, inp["y"], smask, adv, ref, lp_s, lse_s, w.B, w.L,
                                      BETA, 1.0, w.chunk)
    torch.cuda.synchronize()

    W64 = _oracle_w(inp["W"])
    y = inp["y"].cpu().numpy().astype(np.int64)
    mask = inp["mask"].cpu().numpy()
    A = oracle.group_advantages(inp["rewards"].cpu().numpy(), w.G, EPS)

    def rows64(X, rows):
        return _oracle_deq(X[torch.as_tensor(rows, device="cuda")])

    # dH rows of the dense run
    act = np.nonzero(mask)[0]
    drows = np.array(sorted(set(rng.choice(act, size=256, replace=False).tolist())))
    H64 = np.zeros((w.N, w.d))
    H64[drows] = rows64(inp["H"], drows)
    ref64 = np.zeros(w.N)
    ref64[drows], _ = oracle.token_logprobs(rows64(inp["H_ref"], drows), W64, y[drows])
    o_dH, _ = oracle.loss_backward(H64, W64, y, mask, A, ref64, w.L, BETA, dh_rows=drows,
                                   want_dW=False)
    g_dH = to64(dH[torch.as_tensor(drows, device="cuda")])
    print(f"[fp8-full-bwd] dH rows cos {cosine(g_dH, o_dH):.6f} "
          f"maxrel {max_abs_rel(g_dH, o_dH):.2e}", flush=True)
    assert cosine(g_dH, o_dH) >= 0.999
    assert max_abs_rel(g_dH, o_dH) <= 1e-2
    # full dW of the sparse-mask run
    Hk = np.zeros((w.N, w.d))
    Hk[keep] = rows64(inp["H"], keep)
    refk = np.zeros(w.N)
    refk[keep], _ = oracle.token_logprobs(rows64(inp["H_ref"], keep), W64, y[keep])
    o_dHk, o_dW = oracle.loss_backward(Hk, W64, y, smask.cpu().numpy(), A, refk, w.L, BETA,
                                       dh_rows=keep)
    g_dW = to64(dW_s)
    print(f"[fp8-full-bwd] dW cos {cosine(g_dW, o_dW):.6f} maxrel {max_abs_rel(g_dW, o_dW):.2e}",
          flush=True)
    assert cosine(g_dW, o_dW) >= 0.999
    assert max_abs_rel(g_dW, o_dW) <= 1e-2
    g_dHk = to64(dH_s[torch.as_tensor(keep, device="cuda")])
    assert cosine(g_dHk, o_dHk) >= 0.999
    assert max_abs_rel(g_dHk, o_dHk) <= 1e-2


def _fp8_shapes():
    rng = np.random.RandomState(77)
    out = []
    for k in range(4):
        prompts, G = int(rng.randint(1, 3)), int(rng.randint(1, 5))
        L = int(rng.randint(2, 160))
        lo = int(rng.randint(1, L + 1))
        hi = int(rng.randint(lo, L + 1))
        d = 16 * int(rng.randint(1, 25))            # fp8 rows in whole 16-byte vectors
        V = int(rng.randint(17, 2400))
        chunk = int(rng.choice([int(rng.randint(1, 100)), int(rng.randint(100, 600)), 1 << 14]))
        out.append((f"P{prompts}G{G}L{L}-d{d}-V{V}-c{chunk}",
                    small(prompts=prompts, G=G, L=L, d=d, V=V, chunk=chunk, len_lo=lo,
                          len_hi=hi)))
    return out


FP8_SHAPES = _fp8_shapes()


@pytest.mark.parametrize("case", FP8_SHAPES, ids=[c[0] for c in FP8_SHAPES])
def test_fp8_irregular_shape_matches_oracle(case):
    """A seeded sweep of irregular shapes through the fp8 chain.  The reference
    hidden states are drawn independently of H, so that the KL term is well
    conditioned wherever the advantage term cancels (one generation per
    prompt, or equal masked lengths in a group)."""
    _need_gpu()
    name, w = case
    print(f"[fp8-shape] {name}", flush=True)
    inp = workloads.generate(w, seed=23, device="cuda")
    inp["H_ref"] = workloads.draw_hidden(w.N, w.d, torch.bfloat16, 99, "cuda")
    Hq = gp.quantize_fp8(inp["H"], per_row=True)
    Rq = gp.quantize_fp8(inp["H_ref"], per_row=True)
    Wq = gp.quantize_fp8(inp["W"], per_row=False)
    g = _gpu_chain_fp8(inp, w, Hq, Rq, Wq, w.chunk)
    H, R, W = _oracle_deq(inp["H"]), _oracle_deq(inp["H_ref"]), _oracle_w(inp["W"])
    y = inp["y"].cpu().numpy().astype(np.int64)
    mask = inp["mask"].cpu().numpy()
    A = oracle.group_advantages(inp["rewards"].cpu().numpy(), w.G, EPS)
    o_ref, _ = oracle.token_logprobs(R, W, y)
    o = oracle.loss_forward(H, W, y, mask, A, o_ref, w.L, BETA)
    o_dH, o_dW = oracle.loss_backward(H, W, y, mask, A, o_ref, w.L, BETA, 1.0)
    assert np.abs(to64(g["ref"]) - o_ref).max() <= 1e-4
    assert np.abs(to64(g["lp"]) - o["lp"]).max() <= 1e-4
    assert np.abs(to64(g["lse"]) - o["lse"]).max() <= 1e-4
    assert abs(g["loss"].item() - o["loss"]) <= 2e-3 * abs(o["loss"])
    for k, ov in (("dH", o_dH), ("dW", o_dW)):
        assert cosine(to64(g[k]), ov) >= 0.999, k
        assert max_abs_rel(to64(g[k]), ov) <= 1e-2, k
    assert np.all(to64(g["dH"])[~mask.astype(bool)] == 0.0)
