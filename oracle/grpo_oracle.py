"""Float64 CPU oracle for the chunked GRPO policy loss.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The product path
(the HIP library and its Python binding) never does, and this module imports
nothing from it.

It is the plain definition of what the fused GPU path computes, written out in
float64 NumPy with the full logits materialised one block of rows at a time:
no online log-sum-exp, no vocabulary splits, no stored-dZ slabs, no fusion.

Sources (pages as extracted):
  [P-blog]  Unsloth "Long-context GRPO" blog, Chinese translation at
            zjt100.com; sections "Unsloth efficient GRPO algorithm" and
            "GRPO maths and the problems found".
  [P-docs]  Unsloth docs "GRPO with 7x longer context" (French edition);
            sections "Flattened sequence length chunking", "Hidden states
            chunking" and "Offloading activations for log softmax".
  [P-aibit] aibit.im "Mastering GRPO" (French); section "From RLHF and PPO to
            the efficiency of GRPO".

The loss and KL formula images were lost from the pages; what they state in
prose fixes the pieces used here:
  * the policy term multiplies exp(lp - stopgrad(lp)), whose value is 1 and
    whose gradient is that of lp, by the per-sequence advantage broadcast
    over the sequence's tokens [P-blog, GRPO maths];
  * the KL is the reverse KL between the trained policy Q and the frozen
    reference P, estimated without an extra factor of Q, scaled by beta = 0.04
    [P-blog, GRPO maths].  The estimator with that property named there
    (Schulman's) is k3: exp(x) - x - 1 with x = ref_lp - lp;
  * log-probabilities come from float32-or-better logits with the max-shifted
    log-sum-exp [P-docs, flattened chunking, note 2; P-blog, GRPO maths];
  * the advantage is derived per prompt group from the group's rewards
    [P-aibit, From RLHF and PPO]; here (r - mean) / (std + eps), sample std.
Readings where the pages are silent (aggregation, std estimator, masked-token
outputs, empty mask) are listed in the module-level notes of each function.

The pages' four-run ablation [P-blog, GRPO maths] also trains with the detach
removed, with a "full" reverse KL carrying the extra factor of Q, and with a
forward KL; the formulas are lost, and the readings taken here are stated
with each function (token_kl, token_kl_slope, loss_forward).  A per-sequence
mean aggregation (mean over each completion's tokens, then over completions)
is offered beside the global token mean.

Parity unpinned: nothing.  Every function is pinned by the CPU tests against
closed forms, invariants, library routines (scipy log_softmax, numpy std,
torch float64 autograd of the literal policy-term expression) and central
finite differences of the stop-gradient surrogate.  The row-block loop of
loss_backward is pinned with more than one block: on the 512-token tiny
workload (two blocks of 256 rows, against autograd and central differences)
and with 3- and 7-row blocks on a toy problem.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 256


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# advantages
# ---------------------------------------------------------------------------
def group_advantages(rewards, group_size, eps=1e-4):
    """A_b = (r_b - mean_g) / (std_g + eps) within each group of `group_size`.

    [P-aibit, From RLHF and PPO]: GRPO samples several answers per prompt,
    scores each, and turns the scores into an advantage statistically, in
    place of a value model.  Groups are consecutive runs of `group_size`
    rewards.  std is the sample standard deviation (divide by n - 1); a group
    of one has std := 0, so its advantage is 0.  NaN rewards propagate.
    """
    r = _f64(rewards).reshape(-1, group_size)
    n = r.shape[1]
    mean = r.sum(axis=1, keepdims=True) / n
    dev = r - mean
    if n > 1:
        std = np.sqrt((dev * dev).sum(axis=1, keepdims=True) / (n - 1))
    else:
        std = np.zeros_like(mean)
    return (dev / (std + eps)).reshape(-1)


# ---------------------------------------------------------------------------
# log-probabilities
# ---------------------------------------------------------------------------
def logits(H_rows, W):
    """z = H W^T for a block of rows: [b, d] x [V, d] -> [b, V], float64.

    [P-docs, Offloading activations]: the logits of a batch slice are the
    hidden states times the LM head.
    """
    return _f64(H_rows) @ _f64(W).T


def _xform(opts):
    """(s, cap, T) from a logit-transform options dict; 0 (or absent) means off."""
    o = opts or {}
    mul = float(o.get("logit_scale_multiply", 0.0))
    div = float(o.get("logit_scale_divide", 0.0))
    cap = float(o.get("logit_softcapping", 0.0))
    T = float(o.get("temperature", 0.0))
    s = (mul if mul != 0.0 else 1.0) / (div if div != 0.0 else 1.0)
    return s, cap, (T if T != 0.0 else 1.0)


def logit_transform(Z, opts=None):
    """Logits after the optional scale, softcap and temperature, float64.

    [P-docs, Flattened sequence length chunking]: the chunked log-softmax
    takes logit_scale_multiply, logit_scale_divide, logit_softcapping and
    temperature, and its notes say softcapping and temperature are supported.
    The pages give no formulas; the plainest reading, applied in the order of
    the call's arguments: z * multiply, / divide, cap * tanh(z / cap), / T.
    A zero multiply, divide or cap is "off"; a zero temperature means 1.
    """
    s, cap, T = _xform(opts)
    U = _f64(Z) * s
    if cap != 0.0:
        U = cap * np.tanh(U / cap)
    return U / T


def logit_transform_slope(Z, opts=None):
    """d logit_transform(z) / dz, elementwise: (s / T) (1 - tanh^2(s z / cap))."""
    s, cap, T = _xform(opts)
    if cap == 0.0:
        return np.full(np.shape(Z), s / T)
    t = np.tanh(_f64(Z) * s / cap)
    return (s / T) * (1.0 - t * t)


def lse_and_target(Z, y_rows):
    """Max-shifted log-sum-exp of each row of Z and the target log-prob.

    [P-blog, GRPO maths]: the logsumexp trick; lse = M + log sum exp(z - M)
    with M the row max.  lp = z[y] - lse.
    """
    M = Z.max(axis=1)
    lse = M + np.log(np.exp(Z - M[:, None]).sum(axis=1))
    lp = Z[np.arange(Z.shape[0]), np.asarray(y_rows, dtype=np.int64)] - lse
    return lp, lse


def token_logprobs(H, W, y, rows=None, block=ROW_BLOCK, opts=None):
    """(lp, lse) for every token (or for the listed `rows`), float64.

    [P-docs, Flattened sequence length chunking]: the selective log-softmax
    of the hidden states through the LM head, gathered at the completion ids.
    The logits of `block` rows are formed in full, transformed (`opts`, see
    logit_transform), then reduced.
    """
    H = np.asarray(H)
    y = np.asarray(y)
    idx = np.arange(H.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    lp = np.empty(len(idx))
    lse = np.empty(len(idx))
    for b0 in range(0, len(idx), block):
        sel = idx[b0:b0 + block]
        Z = logits(H[sel], W)
        if opts:
            Z = logit_transform(Z, opts)
        lp[b0:b0 + block], lse[b0:b0 + block] = lse_and_target(Z, y[sel])
    return lp, lse


# ---------------------------------------------------------------------------
# fp8 (e4m3) inputs
# ---------------------------------------------------------------------------
# [P-docs, introduction and "Getting started"]: FP8 RL training is offered
# (an FP8 GRPO notebook), and [P-blog, Unsloth efficient GRPO algorithm] warns
# that a naive linear cross-entropy under float8 mixed precision breaks loss
# scaling.  No recipe is given.  Reading: the LM-head GEMM takes float8 e4m3
# operands (the OCP "fn" variant: 4 exponent bits with bias 7, 3 mantissa
# bits, no infinities, S.1111.111 is NaN, largest finite 448) with float32
# accumulation and float32 log-sum-exp; each hidden-state row (token) has its
# own scale and the head one scale; scales are powers of two, so dequantised
# values are exact and only the e4m3 rounding decides a code.
FP8_MAX = 448.0


def fp8_e4m3_decode(codes):
    """Value of each e4m3fn code, float64 (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def _fp8_positive_table():
    """The 127 finite non-negative e4m3fn values, ascending, and their codes."""
    codes = np.arange(0, 127, dtype=np.uint8)
    return fp8_e4m3_decode(codes), codes


def fp8_e4m3_encode(x):
    """Nearest e4m3fn code to each float64 x with |x| <= 448, ties to the even
    code (even mantissa); the sign bit follows the sign of x, zero included."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > FP8_MAX):
        raise ValueError("fp8_e4m3_encode needs finite |x| <= 448")
    vals, codes = _fp8_positive_table()
    a = np.abs(x).reshape(-1)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(codes[lo] % 2 == 0, lo, hi)))
    out = codes[pick].astype(np.uint8)
    neg = np.signbit(x.reshape(-1))
    out = np.where(neg, out | 0x80, out).astype(np.uint8)
    return out.reshape(x.shape)


def fp8_scale_exponent(absmax):
    """Smallest integer e with absmax <= 448 * 2**e (0 for absmax = 0)."""
    a = float(absmax)
    if a == 0.0:
        return 0
    f, k = np.frexp(a)           # a = f 2^k, 0.5 <= f < 1; 448 = 0.875 2^9
    return int(k - 9) if f <= 0.875 else int(k - 8)


def fp8_quantize(X, per_row=True):
    """(codes uint8 [rows, cols], scales float64 [rows] or [1]): X ~ codes * scale.

    The scale of a row (or of the whole tensor) is 2**e with e from
    fp8_scale_exponent of its largest |x|; codes = e4m3 rounding of x / 2**e,
    an exact division, so |x / scale| <= 448 and only the rounding is inexact.
    """
    X = _f64(X)
    if per_row:
        e = np.array([fp8_scale_exponent(np.abs(r).max() if r.size else 0.0) for r in X])
    else:
        e = np.array([fp8_scale_exponent(np.abs(X).max() if X.size else 0.0)])
    sc = np.exp2(e.astype(np.float64))
    codes = fp8_e4m3_encode(X / (sc[:, None] if per_row else sc[0]))
    return codes, sc


def fp8_dequantize(codes, scales):
    """codes * scale per row (scales of length rows) or for the tensor (length 1)."""
    v = fp8_e4m3_decode(codes)
    s = _f64(scales)
    return v * (s[:, None] if s.size > 1 or v.shape[0] == 1 else s[0])


# ---------------------------------------------------------------------------
# per-token KL and loss
# ---------------------------------------------------------------------------
def reverse_kl_k3(ref_lp, lp):
    """kl = exp(x) - x - 1 with x = ref_lp - lp (unscaled, every token).

    [P-blog, GRPO maths]: reverse KL with Q the trained policy and P the
    reference, estimated without an extra factor of Q.
    """
    x = _f64(ref_lp) - _f64(lp)
    return np.exp(x) - x - 1.0


def forward_kl(ref_lp, lp):
    """kl = r log r - (r - 1) with r = exp(ref_lp - lp) (unscaled, every token).

    [P-blog, GRPO maths]: the ablation's forward-KL run, KL(P || Q) with P the
    reference.  The tokens are drawn from Q, so the estimator weights by
    r = P / Q: r log r - (r - 1) has expectation KL(P || Q) under Q (the r - 1
    term has mean zero) and is >= 0 pointwise, the forward-direction
    counterpart of k3 in the estimator family of Schulman's note that the
    pages cite.
    """
    x = _f64(ref_lp) - _f64(lp)
    r = np.exp(x)
    return r * x - (r - 1.0)


def reverse_kl_q(ref_lp, lp):
    """kl = q (exp(x) - x - 1), x = ref_lp - lp, q = exp(lp) (every token).

    [P-blog, GRPO maths]: the ablation's "full reverse KL", the k3 term with
    the extra factor of Q (the trained policy's probability of the sampled
    token) that the pages' derivation found missing.  Plainest reading: the
    factor multiplies the per-token term and is differentiated with it.
    """
    return np.exp(_f64(lp)) * reverse_kl_k3(ref_lp, lp)


KL_ESTIMATORS = ("reverse", "forward", "reverse_q")


def _variant(opts):
    """(kl estimator index, detach removed, per-sequence mean) of an options dict."""
    o = opts or {}
    return int(o.get("kl_estimator", 0)), bool(o.get("no_detach", 0)), int(o.get("aggregation", 0))


def token_kl(ref_lp, lp, opts=None):
    """Per-token KL of the estimator that `opts["kl_estimator"]` names:
    0 reverse k3 (the default), 1 forward, 2 reverse with the factor Q."""
    k = _variant(opts)[0]
    if k == 0:
        return reverse_kl_k3(ref_lp, lp)
    if k == 1:
        return forward_kl(ref_lp, lp)
    if k == 2:
        return reverse_kl_q(ref_lp, lp)
    raise ValueError(f"unknown kl_estimator {k}")


def token_kl_slope(ref_lp, lp, opts=None):
    """d token_kl / d lp, elementwise (x = ref_lp - lp, so dx/dlp = -1):
    k3: 1 - exp(x);  forward: -x exp(x);  reverse with Q: q (k3 + 1 - exp(x)) = -x q."""
    k = _variant(opts)[0]
    x = _f64(ref_lp) - _f64(lp)
    if k == 0:
        return 1.0 - np.exp(x)
    if k == 1:
        return -x * np.exp(x)
    if k == 2:
        return -x * np.exp(_f64(lp))
    raise ValueError(f"unknown kl_estimator {k}")


def token_weights(mask, seq_len, opts=None):
    """w_t with loss = sum_t w_t l_t.

    Global token mean (the default): w_t = m_t / max(sum m, 1), one mean over
    all unmasked flattened tokens.  Per-sequence mean (`aggregation` 1):
    w_t = m_t / (B max(n_b, 1)) with n_b the unmasked tokens of t's sequence,
    i.e. each completion's masked mean, then the plain mean over all B
    completions (an empty completion contributes 0 and still counts in B).
    """
    m = _f64(mask)
    if _variant(opts)[2] == 1:
        mb = m.reshape(-1, seq_len)
        n = mb.sum(axis=1, keepdims=True)
        return (mb / (mb.shape[0] * np.maximum(n, 1.0))).reshape(-1)
    return m / max(m.sum(), 1.0)


def token_advantages(adv, seq_len):
    """A per flattened token: sequence b's advantage on its seq_len tokens.

    [P-blog, GRPO maths]: the advantages are unsqueezed along the sequence
    axis, so one value covers all tokens of a completion.
    """
    return np.repeat(_f64(adv), seq_len)


def loss_forward(H, W, y, mask, adv, ref_lp, seq_len, beta=0.04, opts=None):
    """Masked GRPO loss plus the per-token outputs.

    l_t = -(R_t * A_t - beta * kl_t), with R_t = exp(lp_t - stopgrad(lp_t)),
    whose value is exactly 1 [P-blog, GRPO maths]; with the detach removed
    (`no_detach`) R_t = exp(lp_t - lp_t), still 1 in value.
    kl_t is token_kl (reverse k3 unless `kl_estimator` says otherwise).
    loss = sum_t w_t l_t with w from token_weights: by default the mean over
    all unmasked flattened tokens (an empty mask gives 0).
    lp, kl and lse are reported for every token, masked or not.
    """
    lp, lse = token_logprobs(H, W, y, opts=opts)
    kl = token_kl(ref_lp, lp, opts)
    A_t = token_advantages(adv, seq_len)
    R = 1.0
    ell = -(R * A_t - beta * kl)
    loss = (token_weights(mask, seq_len, opts) * ell).sum()
    return dict(loss=float(loss), lp=lp, kl=kl, lse=lse, ell=ell)


def loss_coefficients(mask, adv, ref_lp, lp, seq_len, beta=0.04, grad_loss=1.0, opts=None):
    """c_t = d loss / d lp_t.

    From l_t = -(R_t A_t - beta kl_t): with the detach, dR/dlp = R = 1; with
    it removed, R = exp(lp - lp) is constant and dR/dlp = 0, so the advantage
    term carries no gradient [P-blog, GRPO maths: removing the detach broke
    training].  dkl/dlp is token_kl_slope (1 - exp(x) for k3).  The
    aggregation contributes w_t (token_weights); grad_loss is the upstream
    scalar.
    """
    A_t = token_advantages(adv, seq_len)
    dR = 0.0 if _variant(opts)[1] else 1.0
    w = token_weights(mask, seq_len, opts)
    return grad_loss * w * (-dR * A_t + beta * token_kl_slope(ref_lp, lp, opts))


def loss_backward(H, W, y, mask, adv, ref_lp, seq_len, beta=0.04, grad_loss=1.0,
                  dh_rows=None, want_dW=True, block=ROW_BLOCK, opts=None):
    """Gradients of the loss w.r.t. H and W, float64.

    [P-docs, Offloading activations]: the backward recomputes the logits of
    each slice instead of keeping them from the forward.  Per token:
      p_t = softmax(f(z_t));  dZ_t = c_t (onehot(y_t) - p_t) f'(z_t)
      dH_t = dZ_t W;          dW = sum_t dZ_t^T h_t
    with f the logit transform of `opts` (the identity without it).
    Returns (dH, dW).  dH has one row per entry of `dh_rows` (all tokens if
    None).  dW is the value the GPU adds to its accumulator (None when
    want_dW is False).  Only unmasked tokens contribute to dW (c_t = 0
    elsewhere), so only they and the requested dH rows are visited.
    """
    H = np.asarray(H)
    y = np.asarray(y)
    N = H.shape[0]
    Wf = _f64(W)
    mask = np.asarray(mask)
    lp_all = np.zeros(N)
    active = np.nonzero(mask)[0]
    rows = np.arange(N) if dh_rows is None else np.asarray(dh_rows, dtype=np.int64)
    need = np.union1d(active, rows) if want_dW else np.unique(rows)
    # per-token coefficient needs lp of the token: recompute from full logits
    lp_need, _ = token_logprobs(H, W, y, rows=need, block=block, opts=opts)
    lp_all[need] = lp_need
    c = loss_coefficients(mask, adv, ref_lp, lp_all, seq_len, beta, grad_loss, opts)
    dW = np.zeros_like(Wf)
    dH = np.zeros((len(rows), Wf.shape[1]))
    pos = {int(t): i for i, t in enumerate(rows)}
    for b0 in range(0, len(need), block):
        sel = need[b0:b0 + block]
        Hs = _f64(H[sel])
        Z = Hs @ Wf.T
        Zf = logit_transform(Z, opts)
        M = Zf.max(axis=1, keepdims=True)
        P = np.exp(Zf - M)
        P /= P.sum(axis=1, keepdims=True)
        dZ = -P
        dZ[np.arange(len(sel)), y[sel].astype(np.int64)] += 1.0
        dZ *= c[sel][:, None]
        dZ *= logit_transform_slope(Z, opts)
        if want_dW:
            dW += dZ.T @ Hs
        g = dZ @ Wf
        for i, t in enumerate(sel):
            j = pos.get(int(t))
            if j is not None:
                dH[j] = g[i]
    return dH, (dW if want_dW else None)
