"""Pins for the float64 oracle: closed forms, invariants, library routines,
brute force and finite differences.  Each test is chosen so a plausible slip
in the oracle (a dropped term, a wrong sign or index, a transposed operand,
the wrong std estimator) fails at least one of them.  CPU only."""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from workloads import BY_NAME

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BETA = 0.04


def _table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _problem(seed=0, P=2, G=3, L=5, d=7, V=11, ref_sigma=0.05, lo=2, hi=5):
    rng = np.random.default_rng(seed)
    B = P * G
    N = B * L
    H = rng.standard_normal((N, d))
    W = 0.3 * rng.standard_normal((V, d))
    H_ref = H + ref_sigma * rng.standard_normal((N, d))
    y = rng.integers(0, V, N)
    r = rng.integers(0, 4, B).astype(np.float64)
    lengths = rng.integers(lo, hi + 1, B)
    mask = (np.arange(L)[None, :] < lengths[:, None]).astype(np.uint8).reshape(-1)
    adv = oracle.group_advantages(r, G)
    ref_lp, _ = oracle.token_logprobs(H_ref, W, y)
    return dict(H=H, W=W, H_ref=H_ref, y=y, r=r, mask=mask, adv=adv, ref_lp=ref_lp,
                L=L, G=G, N=N, V=V, d=d)


# --------------------------------------------------------------------------- advantages
def test_advantages_closed_form_golden():
    rows = _table("advantages_closed_form.txt")
    r = np.array([float(a) for a, _ in rows])
    want = np.array([float(b) for _, b in rows])
    got = oracle.group_advantages(r, 4, eps=1e-4)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_advantages_match_numpy_std_ddof1():
    rng = np.random.default_rng(3)
    r = rng.integers(0, 4, (6, 8)).astype(np.float64)
    want = (r - r.mean(axis=1, keepdims=True)) / (np.std(r, axis=1, ddof=1, keepdims=True) + 1e-4)
    np.testing.assert_allclose(oracle.group_advantages(r.reshape(-1), 8), want.reshape(-1),
                               rtol=1e-14, atol=1e-14)


def test_advantages_group_sums_vanish():
    rng = np.random.default_rng(4)
    r = rng.standard_normal(40)
    A = oracle.group_advantages(r, 5).reshape(8, 5)
    assert np.abs(A.sum(axis=1)).max() < 1e-12


def test_advantages_degenerate_groups():
    assert np.all(oracle.group_advantages(np.full(8, 2.0), 4) == 0.0)
    assert np.all(oracle.group_advantages(np.array([0.0, 3.0, 1.0]), 1) == 0.0)
    A = oracle.group_advantages(np.array([1.0, np.nan, 2.0, 3.0, 0.0, 1.0, 2.0, 3.0]), 4)
    assert np.all(np.isnan(A[:4])) and np.all(np.isfinite(A[4:]))


# --------------------------------------------------------------------------- log-probs
def test_logprobs_match_scipy_log_softmax():
    p = _problem(1)
    lp, lse = oracle.token_logprobs(p["H"], p["W"], p["y"])
    Z = p["H"] @ p["W"].T
    want = scipy.special.log_softmax(Z, axis=1)[np.arange(p["N"]), p["y"]]
    np.testing.assert_allclose(lp, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(Z, axis=1), rtol=1e-13)
    assert np.all(lp <= 0) and np.all(lse >= Z.max(axis=1))


def test_logprobs_brute_force_python_loops():
    rng = np.random.default_rng(2)
    H = rng.standard_normal((3, 4))
    W = rng.standard_normal((5, 4))
    y = [4, 0, 2]
    lp, _ = oracle.token_logprobs(H, W, y)
    for t in range(3):
        z = [sum(H[t][k] * W[v][k] for k in range(4)) for v in range(5)]
        want = z[y[t]] - math.log(sum(math.exp(zv) for zv in z))
        assert abs(lp[t] - want) < 1e-13


def test_logprobs_closed_forms():
    # W = 0: every logit is 0, so lp = -log V and lse = log V.
    H = np.ones((4, 3))
    lp, lse = oracle.token_logprobs(H, np.zeros((7, 3)), [0, 3, 6, 2])
    np.testing.assert_allclose(lp, -math.log(7), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(7), rtol=0, atol=1e-15)
    # V = 2, logits (a, b): lp of target 0 is -log(1 + exp(b - a)).
    H = np.array([[1.0, 0.0], [0.0, 1.0]])
    W = np.array([[0.7, -0.2], [-1.3, 2.5]])       # z_0 = (0.7, -1.3), z_1 = (-0.2, 2.5)
    lp, _ = oracle.token_logprobs(H, W, [0, 0])
    np.testing.assert_allclose(lp, [-math.log1p(math.exp(-2.0)), -math.log1p(math.exp(2.7))],
                               rtol=1e-15)


def test_logprobs_large_logits_stay_finite():
    # max shift: logits near 1e3 must not overflow
    H = np.array([[1000.0], [-1000.0]])
    W = np.array([[1.0], [0.999]])
    lp, _ = oracle.token_logprobs(H, W, [0, 1])
    np.testing.assert_allclose(lp, [-math.log1p(math.exp(-1.0)), -math.log1p(math.exp(-1.0))],
                               rtol=1e-12)


def test_logprobs_block_size_and_row_subset_invariance():
    p = _problem(5, P=3, G=4, L=9)
    a, _ = oracle.token_logprobs(p["H"], p["W"], p["y"], block=256)
    b, _ = oracle.token_logprobs(p["H"], p["W"], p["y"], block=7)
    rows = np.array([5, 0, 17, 100])
    c, _ = oracle.token_logprobs(p["H"], p["W"], p["y"], rows=rows, block=3)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a[rows], c)


# --------------------------------------------------------------------------- KL
def test_kl_closed_form_golden():
    for x, want in _table("kl_closed_form.txt"):
        x, want = float(x), float(want)
        # x = ref_lp - lp: put ref_lp = x + lp for a non-trivial lp
        got = oracle.reverse_kl_k3(np.array([x - 2.5]), np.array([-2.5]))[0]
        assert abs(got - want) < 1e-15, (x, got, want)


def test_kl_nonnegative_and_zero_only_at_equality():
    rng = np.random.default_rng(6)
    ref = -rng.random(1000) * 10
    lp = -rng.random(1000) * 10
    kl = oracle.reverse_kl_k3(ref, lp)
    assert np.all(kl >= 0) and np.all(kl > 0)
    assert np.all(oracle.reverse_kl_k3(lp, lp) == 0.0)


# --------------------------------------------------------------------------- loss
def test_policy_equals_reference_gives_zero_kl_and_minus_mean_advantage():
    p = _problem(7)
    ref_lp, _ = oracle.token_logprobs(p["H"], p["W"], p["y"])      # H_ref = H
    out = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], p["adv"], ref_lp, p["L"], BETA)
    assert np.all(out["kl"] == 0.0)
    A_t = np.repeat(p["adv"], p["L"])
    m = p["mask"].astype(np.float64)
    assert out["loss"] == pytest.approx(-(m * A_t).sum() / m.sum(), rel=1e-15, abs=1e-15)


def test_loss_special_cases():
    p = _problem(8)
    m = p["mask"].astype(np.float64)
    A_t = np.repeat(p["adv"], p["L"])
    # beta = 0: the KL drops out, independent of H and W
    out0 = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"], 0.0)
    assert out0["loss"] == pytest.approx(-(m * A_t).sum() / m.sum(), rel=1e-14)
    # A = 0: loss is beta times the masked mean KL
    zeros = np.zeros_like(p["adv"])
    outa = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], zeros, p["ref_lp"], p["L"], BETA)
    assert outa["loss"] == pytest.approx(BETA * (m * outa["kl"]).sum() / m.sum(), rel=1e-14)
    assert outa["loss"] > 0
    # empty mask: loss 0
    oute = oracle.loss_forward(p["H"], p["W"], p["y"], np.zeros_like(p["mask"]), p["adv"],
                               p["ref_lp"], p["L"], BETA)
    assert oute["loss"] == 0.0


def _torch_autograd_loss(p, H, W, beta=BETA):
    """Independent reference: torch float64 autograd of the stop-gradient ratio
    exp(lp - sg(lp)) times the per-sequence advantage, plus beta times the k3
    KL, masked token mean."""
    B, L = len(p["adv"]), p["L"]
    logp = torch.log_softmax(H @ W.T, dim=1)
    lp = logp[torch.arange(logp.shape[0]), torch.as_tensor(p["y"]).long()].reshape(B, L)
    ratio = (lp - lp.detach()).exp()
    A_tok = torch.as_tensor(p["adv"]).reshape(B, 1).expand(B, L)
    x = torch.as_tensor(p["ref_lp"]).reshape(B, L) - lp
    k3 = x.exp() - x - 1.0
    m = torch.as_tensor(p["mask"]).double().reshape(B, L)
    per_token = beta * k3 - ratio * A_tok
    return (per_token * m).sum() / torch.clamp(m.sum(), min=1.0)


def test_gradients_match_torch_autograd():
    p = _problem(9)
    H = torch.tensor(p["H"], requires_grad=True)
    W = torch.tensor(p["W"], requires_grad=True)
    loss = _torch_autograd_loss(p, H, W)
    loss.backward()
    out = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"], BETA)
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-13)
    dH, dW = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                  p["L"], BETA)
    np.testing.assert_allclose(dH, H.grad.numpy(), rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-10, atol=1e-15)


def _surrogate(p, H, W, lp0, beta=BETA):
    """J = sum m [-(exp(lp - lp0) A - beta kl)] / sum m, lp0 frozen: value equals the
    loss at lp = lp0 and its gradient equals the loss gradient."""
    lp, _ = oracle.token_logprobs(H, W, p["y"])
    A_t = np.repeat(p["adv"], p["L"])
    x = p["ref_lp"] - lp
    ell = -(np.exp(lp - lp0) * A_t - beta * (np.exp(x) - x - 1))
    m = p["mask"].astype(np.float64)
    return (m * ell).sum() / max(m.sum(), 1.0)


@pytest.mark.parametrize("beta,zero_adv", [(BETA, False), (BETA, True), (0.0, False)])
def test_gradients_match_central_differences_of_surrogate(beta, zero_adv):
    p = _problem(10, ref_sigma=0.7)
    if zero_adv:
        p["adv"] = np.zeros_like(p["adv"])          # pure KL path
    lp0, _ = oracle.token_logprobs(p["H"], p["W"], p["y"])
    dH, dW = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                  p["L"], beta)
    rng = np.random.default_rng(11)
    h = 1e-6
    for _ in range(12):
        t, k = rng.integers(0, p["N"]), rng.integers(0, p["d"])
        Hp, Hm = p["H"].copy(), p["H"].copy()
        Hp[t, k] += h
        Hm[t, k] -= h
        fd = (_surrogate(p, Hp, p["W"], lp0, beta) - _surrogate(p, Hm, p["W"], lp0, beta)) / (2 * h)
        assert abs(fd - dH[t, k]) < 1e-8 + 1e-6 * abs(fd), (t, k, fd, dH[t, k])
        v, k = rng.integers(0, p["V"]), rng.integers(0, p["d"])
        Wp, Wm = p["W"].copy(), p["W"].copy()
        Wp[v, k] += h
        Wm[v, k] -= h
        fd = (_surrogate(p, p["H"], Wp, lp0, beta) - _surrogate(p, p["H"], Wm, lp0, beta)) / (2 * h)
        assert abs(fd - dW[v, k]) < 1e-8 + 1e-6 * abs(fd), (v, k, fd, dW[v, k])


def test_gradient_invariants():
    p = _problem(12)
    dH, dW = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                  p["L"], BETA)
    # each dZ row sums to zero, so the vocab-sum of dW vanishes
    assert np.abs(dW.sum(axis=0)).max() < 1e-15 * max(1.0, np.abs(dW).max()) + 1e-16
    # masked tokens get no gradient
    assert np.all(dH[p["mask"] == 0] == 0.0)
    assert np.abs(dH[p["mask"] == 1]).max() > 0
    # requested rows only / no dW
    rows = np.array([3, 0, 11])
    dHr, none = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                     p["L"], BETA, dh_rows=rows, want_dW=False)
    assert none is None
    np.testing.assert_allclose(dHr, dH[rows], rtol=1e-13, atol=1e-18)


def test_policy_equals_reference_gradient_is_weighted_cross_entropy():
    p = _problem(13)
    p["ref_lp"], _ = oracle.token_logprobs(p["H"], p["W"], p["y"])    # H_ref = H
    dH, dW = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                  p["L"], BETA)
    H = torch.tensor(p["H"], requires_grad=True)
    W = torch.tensor(p["W"], requires_grad=True)
    ce = torch.nn.functional.cross_entropy(H @ W.T, torch.as_tensor(p["y"]).long(), reduction="none")
    m = torch.as_tensor(p["mask"]).double()
    w = m * torch.as_tensor(np.repeat(p["adv"], p["L"])) / m.sum()
    (w * ce).sum().backward()
    np.testing.assert_allclose(dH, H.grad.numpy(), rtol=1e-10, atol=1e-16)
    np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-10, atol=1e-16)


# --------------------------------------------------------------------------- multi-block backward
# loss_backward visits its rows in blocks of ROW_BLOCK = 256; the tiny workload
# (2 prompts x 4 generations x 64 tokens, d 256, V 1024) has 512 flattened tokens,
# so these pins run the block loop twice with active tokens in both blocks.
def _tiny_problem():
    from workloads import BY_NAME, generate

    w = BY_NAME["tiny-f32"]
    inp = generate(w, seed=3, device="cpu")
    f64 = lambda t: t.double().numpy()   # noqa: E731
    H, W, H_ref = f64(inp["H"]), f64(inp["W"]), f64(inp["H_ref"])
    y = inp["y"].numpy().astype(np.int64)
    mask = inp["mask"].numpy()
    adv = oracle.group_advantages(inp["rewards"].numpy(), w.G)
    ref_lp, _ = oracle.token_logprobs(H_ref, W, y)
    p = dict(H=H, W=W, H_ref=H_ref, y=y, mask=mask, adv=adv, ref_lp=ref_lp, L=w.L, G=w.G,
             N=w.N, V=w.V, d=w.d)
    assert w.N == 2 * 256          # the oracle's default row block
    assert mask[:w.N // 2].any() and mask[w.N // 2:].any()
    return p


def test_tiny_config_gradients_match_torch_autograd_across_row_blocks():
    p = _tiny_problem()
    H = torch.tensor(p["H"], requires_grad=True)
    W = torch.tensor(p["W"], requires_grad=True)
    _torch_autograd_loss(p, H, W).backward()
    dH, dW = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                  p["L"], BETA)
    np.testing.assert_allclose(dH, H.grad.numpy(), rtol=1e-10, atol=1e-14 * np.abs(dH).max())
    np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-10, atol=1e-14 * np.abs(dW).max())


def test_tiny_config_gradients_match_central_differences():
    """Central differences of the stop-gradient surrogate on the 512-token tiny
    workload: along one random direction over all of H and all of W (the
    directional derivative <dX, U> sums every token's share, so each row block
    must contribute), and at single entries in both row blocks."""
    p = _tiny_problem()
    lp0, _ = oracle.token_logprobs(p["H"], p["W"], p["y"])
    dH, dW = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                  p["L"], BETA)
    rng = np.random.default_rng(15)
    h = 1e-6
    UH = rng.standard_normal(p["H"].shape)
    UW = rng.standard_normal(p["W"].shape)
    fd = (_surrogate(p, p["H"] + h * UH, p["W"], lp0) -
          _surrogate(p, p["H"] - h * UH, p["W"], lp0)) / (2 * h)
    assert abs(fd - (dH * UH).sum()) < 1e-6 * abs(fd) + 1e-9, (fd, (dH * UH).sum())
    fd = (_surrogate(p, p["H"], p["W"] + h * UW, lp0) -
          _surrogate(p, p["H"], p["W"] - h * UW, lp0)) / (2 * h)
    assert abs(fd - (dW * UW).sum()) < 1e-6 * abs(fd) + 1e-9, (fd, (dW * UW).sum())
    active = np.nonzero(p["mask"])[0]
    for t in (active[0], active[-1]):                 # first and second row block
        k = rng.integers(0, p["d"])
        Hp, Hm = p["H"].copy(), p["H"].copy()
        Hp[t, k] += h
        Hm[t, k] -= h
        fd = (_surrogate(p, Hp, p["W"], lp0) - _surrogate(p, Hm, p["W"], lp0)) / (2 * h)
        assert abs(fd - dH[t, k]) < 1e-8 + 1e-6 * abs(fd), (t, k, fd, dH[t, k])
    for v in (p["y"][active[0]], p["y"][active[-1]], rng.integers(0, p["V"])):
        k = rng.integers(0, p["d"])
        Wp, Wm = p["W"].copy(), p["W"].copy()
        Wp[v, k] += h
        Wm[v, k] -= h
        fd = (_surrogate(p, p["H"], Wp, lp0) - _surrogate(p, p["H"], Wm, lp0)) / (2 * h)
        assert abs(fd - dW[v, k]) < 1e-8 + 1e-6 * abs(fd), (v, k, fd, dW[v, k])


def test_backward_row_block_size_and_requested_rows():
    """Small row blocks (7 rows: five blocks on the 30-token problem) give the
    one-block result and torch autograd's; dW does not depend on which dH rows
    are requested (it sums every unmasked token, requested or not)."""
    p = _problem(16)
    one = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"],
                               BETA)
    many = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"],
                                BETA, block=7)
    for a, b in zip(one, many):
        np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-15 * np.abs(a).max())
    H = torch.tensor(p["H"], requires_grad=True)
    W = torch.tensor(p["W"], requires_grad=True)
    _torch_autograd_loss(p, H, W).backward()
    np.testing.assert_allclose(many[0], H.grad.numpy(), rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(many[1], W.grad.numpy(), rtol=1e-10, atol=1e-15)
    masked = np.nonzero(p["mask"] == 0)[0]
    rows = np.array([masked[0], np.nonzero(p["mask"])[0][1]])   # one masked, one active
    dHr, dWr = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                    p["L"], BETA, dh_rows=rows, block=3)
    np.testing.assert_allclose(dWr, one[1], rtol=1e-12, atol=1e-15 * np.abs(one[1]).max())
    np.testing.assert_allclose(dHr, one[0][rows], rtol=1e-12, atol=1e-18)


def test_grad_loss_scales_linearly():
    p = _problem(14)
    a = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"], BETA)
    b = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"], BETA,
                             grad_loss=-2.5)
    for got, base in ((b[0], a[0]), (b[1], a[1])):
        np.testing.assert_allclose(got, -2.5 * base, rtol=1e-13, atol=1e-14 * np.abs(base).max())


# --------------------------------------------------------------------------- logit transforms
XFORMS = [
    {"temperature": 0.7},
    {"logit_softcapping": 1.5},
    {"logit_scale_multiply": 1.3, "logit_scale_divide": 0.8, "logit_softcapping": 2.0,
     "temperature": 1.25},
]


def test_transform_off_is_the_identity():
    p = _problem(20)
    Z = oracle.logits(p["H"], p["W"])
    zero = {"logit_scale_multiply": 0.0, "logit_scale_divide": 0.0, "logit_softcapping": 0.0,
            "temperature": 0.0}
    assert np.array_equal(oracle.logit_transform(Z, zero), Z)
    assert np.array_equal(oracle.logit_transform_slope(Z, zero), np.ones_like(Z))


def test_temperature_is_log_softmax_of_scaled_logits():
    p = _problem(21)
    T = 0.7
    lp, lse = oracle.token_logprobs(p["H"], p["W"], p["y"], opts={"temperature": T})
    Z = (p["H"] @ p["W"].T) / T
    want = scipy.special.log_softmax(Z, axis=1)[np.arange(p["N"]), p["y"]]
    np.testing.assert_allclose(lp, want, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(Z, axis=1), rtol=1e-13)


def test_scale_divide_and_temperature_are_the_same_linear_map():
    p = _problem(22)
    a, _ = oracle.token_logprobs(p["H"], p["W"], p["y"], opts={"logit_scale_multiply": 2.0})
    b, _ = oracle.token_logprobs(p["H"], p["W"], p["y"], opts={"logit_scale_divide": 0.5})
    c, _ = oracle.token_logprobs(p["H"], p["W"], p["y"], opts={"temperature": 0.5})
    d, _ = oracle.token_logprobs(2.0 * p["H"], p["W"], p["y"])
    for got in (b, c, d):
        np.testing.assert_allclose(got, a, rtol=1e-12, atol=1e-13)


def test_softcap_bounds_closed_form_and_large_cap_limit():
    Z = np.linspace(-500.0, 500.0, 2001).reshape(1, -1)
    cap, T = 30.0, 2.0
    f = oracle.logit_transform(Z, {"logit_softcapping": cap, "temperature": T})
    assert np.all(np.abs(f) < cap / T)
    assert np.all(np.diff(f) > 0)                                     # monotone
    z = cap * math.atanh(0.5)                                        # tanh(z / cap) = 1/2
    assert oracle.logit_transform(np.array([[z]]), {"logit_softcapping": cap})[0, 0] == \
        pytest.approx(cap / 2, rel=1e-14)
    assert oracle.logit_transform_slope(np.array([[z]]), {"logit_softcapping": cap})[0, 0] == \
        pytest.approx(0.75, rel=1e-14)                               # 1 - tanh^2
    small = np.linspace(-3, 3, 13).reshape(1, -1)
    np.testing.assert_allclose(oracle.logit_transform(small, {"logit_softcapping": 1e7}), small,
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("opts", XFORMS)
def test_transform_gradients_match_central_differences_of_surrogate(opts):
    p = _problem(23, ref_sigma=0.7)
    lp0, _ = oracle.token_logprobs(p["H"], p["W"], p["y"], opts=opts)
    dH, dW = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                  p["L"], BETA, opts=opts)

    def J(H, W):
        lp, _ = oracle.token_logprobs(H, W, p["y"], opts=opts)
        A_t = np.repeat(p["adv"], p["L"])
        x = p["ref_lp"] - lp
        ell = -(np.exp(lp - lp0) * A_t - BETA * (np.exp(x) - x - 1))
        m = p["mask"].astype(np.float64)
        return (m * ell).sum() / max(m.sum(), 1.0)

    rng = np.random.default_rng(24)
    h = 1e-6
    for _ in range(10):
        t, k = rng.integers(0, p["N"]), rng.integers(0, p["d"])
        Hp, Hm = p["H"].copy(), p["H"].copy()
        Hp[t, k] += h
        Hm[t, k] -= h
        fd = (J(Hp, p["W"]) - J(Hm, p["W"])) / (2 * h)
        assert abs(fd - dH[t, k]) < 1e-8 + 1e-6 * abs(fd), (t, k, fd, dH[t, k])
        v, k = rng.integers(0, p["V"]), rng.integers(0, p["d"])
        Wp, Wm = p["W"].copy(), p["W"].copy()
        Wp[v, k] += h
        Wm[v, k] -= h
        fd = (J(p["H"], Wp) - J(p["H"], Wm)) / (2 * h)
        assert abs(fd - dW[v, k]) < 1e-8 + 1e-6 * abs(fd), (v, k, fd, dW[v, k])


@pytest.mark.parametrize("opts", XFORMS)
def test_transform_gradients_match_torch_autograd(opts):
    p = _problem(25)
    H = torch.tensor(p["H"], requires_grad=True)
    W = torch.tensor(p["W"], requires_grad=True)
    mul = opts.get("logit_scale_multiply", 0.0) or 1.0
    div = opts.get("logit_scale_divide", 0.0) or 1.0
    cap = opts.get("logit_softcapping", 0.0)
    T = opts.get("temperature", 0.0) or 1.0
    Z = (H @ W.T) * mul / div
    if cap:
        Z = cap * torch.tanh(Z / cap)
    Z = Z / T
    B, L = len(p["adv"]), p["L"]
    logp = torch.log_softmax(Z, dim=1)
    lp = logp[torch.arange(logp.shape[0]), torch.as_tensor(p["y"]).long()].reshape(B, L)
    ratio = (lp - lp.detach()).exp()
    x = torch.as_tensor(p["ref_lp"]).reshape(B, L) - lp
    m = torch.as_tensor(p["mask"]).double().reshape(B, L)
    per_token = BETA * (x.exp() - x - 1.0) - ratio * torch.as_tensor(p["adv"]).reshape(B, 1)
    loss = (per_token * m).sum() / torch.clamp(m.sum(), min=1.0)
    loss.backward()
    out = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"],
                              BETA, opts=opts)
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-13)
    dH, dW = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                  p["L"], BETA, opts=opts)
    np.testing.assert_allclose(dH, H.grad.numpy(), rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-10, atol=1e-15)


# --------------------------------------------------------------------------- ablation variants
VARIANTS = [
    {"kl_estimator": 1},
    {"kl_estimator": 2},
    {"no_detach": 1},
    {"aggregation": 1},
    {"kl_estimator": 1, "no_detach": 1, "aggregation": 1},
    {"kl_estimator": 2, "temperature": 0.8},
]


def test_kl_estimators_are_unbiased_on_a_small_vocabulary():
    """Averaged over the trained policy Q on a 9-token vocabulary, k3 is exactly
    KL(Q || P) and the forward estimator exactly KL(P || Q) (scipy rel_entr)."""
    rng = np.random.default_rng(40)
    for _ in range(5):
        q = scipy.special.softmax(rng.standard_normal(9) * 1.5)
        p = scipy.special.softmax(rng.standard_normal(9) * 1.5)
        lp, ref = np.log(q), np.log(p)
        rev = (q * oracle.token_kl(ref, lp, {"kl_estimator": 0})).sum()
        fwd = (q * oracle.token_kl(ref, lp, {"kl_estimator": 1})).sum()
        assert rev == pytest.approx(scipy.special.rel_entr(q, p).sum(), rel=1e-12)
        assert fwd == pytest.approx(scipy.special.rel_entr(p, q).sum(), rel=1e-12)
        assert abs(fwd - rev) > 1e-6          # the two directions differ here


def test_kl_variant_closed_forms_golden():
    names = {"forward": 1, "reverse_q": 2}
    for est, q, pr, want in _table("kl_variants_closed_form.txt"):
        lp, ref = np.log([float(q)]), np.log([float(pr)])
        got = oracle.token_kl(ref, lp, {"kl_estimator": names[est]})[0]
        assert got == pytest.approx(float(want), rel=1e-15, abs=1e-16), (est, q, pr)


def test_kl_variants_nonnegative_and_zero_at_equality():
    rng = np.random.default_rng(41)
    ref, lp = -rng.random(1000) * 10, -rng.random(1000) * 10
    for k in (1, 2):
        assert np.all(oracle.token_kl(ref, lp, {"kl_estimator": k}) > 0)
        assert np.all(oracle.token_kl(lp, lp, {"kl_estimator": k}) == 0.0)


def test_token_weights_hand_example():
    # B = 3 completions of L = 3: lengths 2, 1, 0
    mask = np.array([1, 1, 0, 1, 0, 0, 0, 0, 0], dtype=np.uint8)
    np.testing.assert_allclose(oracle.token_weights(mask, 3),
                               [1 / 3, 1 / 3, 0, 1 / 3, 0, 0, 0, 0, 0], rtol=0, atol=1e-16)
    np.testing.assert_allclose(oracle.token_weights(mask, 3, {"aggregation": 1}),
                               [1 / 6, 1 / 6, 0, 1 / 3, 0, 0, 0, 0, 0], rtol=0, atol=1e-16)


def test_sequence_mean_policy_equals_reference_gives_zero_loss():
    """With kl = 0, the per-sequence mean is -mean_b(A_b), which vanishes because
    each group's advantages sum to zero; the token mean weights sequences by
    length and does not vanish for unequal lengths."""
    p = _problem(42, lo=1, hi=5)
    ref_lp, _ = oracle.token_logprobs(p["H"], p["W"], p["y"])
    for k in (0, 1, 2):
        seq = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], p["adv"], ref_lp, p["L"], BETA,
                                  opts={"kl_estimator": k, "aggregation": 1})
        tok = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], p["adv"], ref_lp, p["L"], BETA,
                                  opts={"kl_estimator": k})
        assert np.all(seq["kl"] == 0.0)
        assert abs(seq["loss"]) < 1e-15
        assert abs(tok["loss"]) > 1e-3


def test_no_detach_gradient_is_the_pure_kl_gradient():
    p = _problem(43, ref_sigma=0.5)
    nd = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"],
                              BETA, opts={"no_detach": 1})
    a0 = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], np.zeros_like(p["adv"]),
                              p["ref_lp"], p["L"], BETA)
    np.testing.assert_allclose(nd[0], a0[0], rtol=1e-13, atol=1e-18)
    np.testing.assert_allclose(nd[1], a0[1], rtol=1e-13, atol=1e-18)
    # the value is that of the detached loss
    f = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"], BETA)
    g = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"], BETA,
                            opts={"no_detach": 1})
    assert f["loss"] == g["loss"]


@pytest.mark.parametrize("opts", VARIANTS)
def test_variant_gradients_match_torch_autograd(opts):
    """Torch float64 autograd of each variant written out literally: the ratio
    with or without detach, the estimator's expression, the aggregation."""
    p = _problem(44, ref_sigma=0.5, lo=0, hi=5)
    H = torch.tensor(p["H"], requires_grad=True)
    W = torch.tensor(p["W"], requires_grad=True)
    T = opts.get("temperature", 0.0) or 1.0
    B, L = len(p["adv"]), p["L"]
    logp = torch.log_softmax((H @ W.T) / T, dim=1)
    lp = logp[torch.arange(logp.shape[0]), torch.as_tensor(p["y"]).long()].reshape(B, L)
    ratio = (lp - lp).exp() if opts.get("no_detach") else (lp - lp.detach()).exp()
    x = torch.as_tensor(p["ref_lp"]).reshape(B, L) - lp
    k = opts.get("kl_estimator", 0)
    if k == 0:
        kl = x.exp() - x - 1.0
    elif k == 1:
        kl = x.exp() * x - (x.exp() - 1.0)
    else:
        kl = lp.exp() * (x.exp() - x - 1.0)
    m = torch.as_tensor(p["mask"]).double().reshape(B, L)
    per_token = BETA * kl - ratio * torch.as_tensor(p["adv"]).reshape(B, 1)
    if opts.get("aggregation"):
        loss = ((per_token * m).sum(dim=1) / torch.clamp(m.sum(dim=1), min=1.0)).mean()
    else:
        loss = (per_token * m).sum() / torch.clamp(m.sum(), min=1.0)
    loss.backward()
    out = oracle.loss_forward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"], p["L"],
                              BETA, opts=opts)
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-13)
    np.testing.assert_allclose(out["kl"], kl.detach().numpy().reshape(-1), rtol=1e-12, atol=1e-15)
    dH, dW = oracle.loss_backward(p["H"], p["W"], p["y"], p["mask"], p["adv"], p["ref_lp"],
                                  p["L"], BETA, opts=opts)
    np.testing.assert_allclose(dH, H.grad.numpy(), rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-10, atol=1e-15)


# --------------------------------------------------------------------------- fp8 (e4m3) inputs
def test_fp8_decode_matches_torch_float8_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.tensor(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.fp8_e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))
    assert np.nanmax(got) == oracle.FP8_MAX


def test_fp8_encode_matches_torch_rounding():
    rng = np.random.default_rng(50)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.05, 0.05, 20000),
                        rng.uniform(-0.004, 0.004, 5000), [448.0, -448.0, 0.0, -0.0]])
    want = torch.tensor(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_e4m3_encode(x), want)


def test_fp8_encode_roundtrip_and_hand_worked_ties():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.fp8_e4m3_encode(oracle.fp8_e4m3_decode(codes)), codes)
    for x, c in _table("fp8_e4m3_ties.txt"):
        assert int(oracle.fp8_e4m3_encode(np.array([float(x)]))[0]) == int(c, 16), x
    with pytest.raises(ValueError):
        oracle.fp8_e4m3_encode(np.array([448.5]))


def test_fp8_scale_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(51)
    for a in np.concatenate([rng.lognormal(0, 6, 2000), [1e-30, 3.0, 448.0, 449.0]]):
        e = oracle.fp8_scale_exponent(a)
        assert a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1), a
    for k in range(-20, 21):
        assert oracle.fp8_scale_exponent(448.0 * 2.0 ** k) == k
        assert oracle.fp8_scale_exponent(448.0 * 2.0 ** k * (1 + 2.0 ** -20)) == k + 1
    assert oracle.fp8_scale_exponent(0.0) == 0


def test_fp8_quantize_rows_bound_and_error():
    rng = np.random.default_rng(52)
    X = rng.standard_normal((40, 300)) * np.exp2(rng.integers(-12, 12, (40, 1)))
    X[3] = 0.0
    codes, sc = oracle.fp8_quantize(X, per_row=True)
    assert np.all(np.log2(sc) == np.round(np.log2(sc)))          # powers of two
    assert sc[3] == 1.0 and np.all(codes[3] == 0)
    D = oracle.fp8_dequantize(codes, sc)
    # 3 mantissa bits: half an ulp is 2^-4 of the value (normal) or 2^-10 of the scale
    err = np.abs(D - X)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(X), 2.0 ** -10 * sc[:, None]) * (1 + 1e-12))
    # each row's largest magnitude lands in the top binade (>= 224 after scaling)
    big = np.abs(X).max(axis=1)
    assert np.all((big / sc >= 224.0) | (big == 0))
    # one scale for the tensor
    codes_t, sct = oracle.fp8_quantize(X, per_row=False)
    assert sct.shape == (1,) and sct[0] == sc.max()
    np.testing.assert_array_equal(oracle.fp8_dequantize(codes_t, sct),
                                  oracle.fp8_e4m3_decode(codes_t) * sct[0])


# --------------------------------------------------------------------------- workload shapes
def test_long_context_workload_reproduces_pages_logit_memory():
    """8 x 20480 tokens x 128256 vocab x 4 B is the pages' 78.3 GB of logits;
    one generation at a time is 9.8 GB; the difference is the 68.5 GB saved."""
    w = BY_NAME["llama3.1-8b-20k-bf16"]
    figs = {k: float(v) for k, v in _table("logit_memory_figures.txt")}
    full = w.N * w.V * 4 / 2**30
    one = w.L * w.V * 4 / 2**30
    assert round(full, 1) == figs["full_fp32_logits"]
    assert round(one, 1) == figs["one_generation_fp32_logits"]
    assert round(full - one, 1) == figs["saved"]
