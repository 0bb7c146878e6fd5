"""Planted mistakes: each case edits the oracle's own source (one plausible slip:
a dropped term, a wrong sign, index or estimator, a transposed or misaligned
operand), loads the edited copy in place of the oracle, and runs every pin of
tests/test_oracle_pins.py against it.  At least one pin must fail for every
case, and the unedited source must pass them all.  CPU only; the edits live
in memory, never on disk."""
import inspect
import os
import types

import pytest

import oracle
import oracle.grpo_oracle as grpo_oracle
import tests.test_oracle_pins as pins

SOURCE_PATH = os.path.join(os.path.dirname(grpo_oracle.__file__), "grpo_oracle.py")
PUBLIC = [n for n in dir(oracle) if not n.startswith("_") and inspect.isfunction(getattr(oracle, n))]

# (name, [(text, replacement), ...]): every text must occur exactly once
MUTATIONS = [
    ("advantages: population std (ddof 0)",
     [("std = np.sqrt((dev * dev).sum(axis=1, keepdims=True) / (n - 1))",
       "std = np.sqrt((dev * dev).sum(axis=1, keepdims=True) / n)")]),
    ("advantages: eps under the square root",
     [("return (dev / (std + eps)).reshape(-1)",
       "return (dev / np.sqrt(std * std + eps)).reshape(-1)")]),
    ("advantages: sign flipped",
     [("dev = r - mean", "dev = mean - r")]),
    ("advantages: batch mean instead of group mean",
     [("mean = r.sum(axis=1, keepdims=True) / n",
       "mean = r.mean() + 0.0 * r.sum(axis=1, keepdims=True)")]),
    ("lse: max term dropped",
     [("lse = M + np.log(np.exp(Z - M[:, None]).sum(axis=1))",
       "lse = np.log(np.exp(Z - M[:, None]).sum(axis=1))")]),
    ("lse: no max shift",
     [("lse = M + np.log(np.exp(Z - M[:, None]).sum(axis=1))",
       "lse = np.log(np.exp(Z).sum(axis=1))")]),
    ("target gather off by one",
     [("lp = Z[np.arange(Z.shape[0]), np.asarray(y_rows, dtype=np.int64)] - lse",
       "lp = Z[np.arange(Z.shape[0]), (np.asarray(y_rows, dtype=np.int64) + 1) % Z.shape[1]] - lse")]),
    ("logits against a reordered vocabulary",
     [("return _f64(H_rows) @ _f64(W).T", "return _f64(H_rows) @ _f64(W)[::-1].T")]),
    ("kl: the -1 term dropped",
     [("return np.exp(x) - x - 1.0", "return np.exp(x) - x")]),
    ("kl: x = lp - ref (forward direction)",
     [("x = _f64(ref_lp) - _f64(lp)\n    return np.exp(x) - x - 1.0",
       "x = _f64(lp) - _f64(ref_lp)\n    return np.exp(x) - x - 1.0")]),
    ("kl: quadratic estimator in place of k3",
     [("return np.exp(x) - x - 1.0", "return 0.5 * x * x")]),
    ("token advantages tiled instead of repeated",
     [("return np.repeat(_f64(adv), seq_len)", "return np.tile(_f64(adv), seq_len)")]),
    ("loss: mean over every token, not the unmasked ones",
     [("    return m / max(m.sum(), 1.0)", "    return m / len(m)")]),
    ("loss: KL penalty added instead of subtracted",
     [("ell = -(R * A_t - beta * kl)", "ell = -(R * A_t + beta * kl)")]),
    ("gradient: KL derivative sign",
     [("        return 1.0 - np.exp(x)", "        return np.exp(x) - 1.0")]),
    ("gradient: advantage sign",
     [("(-dR * A_t + beta *", "(dR * A_t + beta *")]),
    ("gradient: mean normalisation dropped",
     [("return grad_loss * w * (", "return grad_loss * _f64(mask) * (")]),
    ("gradient: grad_loss ignored",
     [("return grad_loss * w * (", "return 1.0 * w * (")]),
    ("dZ: p - onehot instead of onehot - p",
     [("dZ = -P\n", "dZ = P.copy()\n"),
      ("dZ[np.arange(len(sel)), y[sel].astype(np.int64)] += 1.0",
       "dZ[np.arange(len(sel)), y[sel].astype(np.int64)] -= 1.0")]),
    ("dZ: softmax normalised over the whole block",
     [("P /= P.sum(axis=1, keepdims=True)", "P /= P.sum()")]),
    ("dZ: onehot at the wrong index",
     [("dZ[np.arange(len(sel)), y[sel].astype(np.int64)] += 1.0",
       "dZ[np.arange(len(sel)), (y[sel].astype(np.int64) + 1) % Wf.shape[0]] += 1.0")]),
    ("dW: hidden rows misaligned with dZ rows",
     [("dW += dZ.T @ Hs", "dW += dZ.T @ Hs[::-1]")]),
    ("dH: vocabulary order of W reversed",
     [("g = dZ @ Wf", "g = dZ @ Wf[::-1]")]),
    ("transform: temperature multiplies instead of divides",
     [("    return U / T\n", "    return U * T\n")]),
    ("transform: softcap without the outer cap factor",
     [("U = cap * np.tanh(U / cap)", "U = np.tanh(U / cap)")]),
    ("transform slope: the 1 - tanh^2 factor dropped",
     [("return (s / T) * (1.0 - t * t)", "return (s / T) * (1.0 + 0.0 * t)")]),
    ("transform slope: 1 / T dropped",
     [("return (s / T) * (1.0 - t * t)", "return s * (1.0 - t * t)")]),
    ("transform: divide applied as a multiply",
     [("s = (mul if mul != 0.0 else 1.0) / (div if div != 0.0 else 1.0)",
       "s = (mul if mul != 0.0 else 1.0) * (div if div != 0.0 else 1.0)")]),
    ("backward: softmax of the raw logits, not the transformed ones",
     [("M = Zf.max(axis=1, keepdims=True)\n        P = np.exp(Zf - M)",
       "M = Z.max(axis=1, keepdims=True)\n        P = np.exp(Z - M)")]),
    ("forward kl: the r - 1 term dropped",
     [("return r * x - (r - 1.0)", "return r * x")]),
    ("forward kl: k3 in its place",
     [("return r * x - (r - 1.0)", "return r - x - 1.0")]),
    ("forward kl: the ratio inverted",
     [("    r = np.exp(x)\n    return r * x - (r - 1.0)", "    r = np.exp(-x)\n    return -r * x - (r - 1.0)")]),
    ("full reverse kl: the factor Q dropped",
     [("return np.exp(_f64(lp)) * reverse_kl_k3(ref_lp, lp)", "return reverse_kl_k3(ref_lp, lp)")]),
    ("full reverse kl: the reference's probability as the factor",
     [("return np.exp(_f64(lp)) * reverse_kl_k3(ref_lp, lp)",
       "return np.exp(_f64(ref_lp)) * reverse_kl_k3(ref_lp, lp)")]),
    ("forward kl slope: sign",
     [("        return -x * np.exp(x)", "        return x * np.exp(x)")]),
    ("full reverse kl slope: the factor Q held constant",
     [("        return -x * np.exp(_f64(lp))", "        return np.exp(_f64(lp)) * (1.0 - np.exp(x))")]),
    ("no-detach switch ignored",
     [("dR = 0.0 if _variant(opts)[1] else 1.0", "dR = 1.0")]),
    ("sequence mean: divided by all unmasked tokens",
     [("return (mb / (mb.shape[0] * np.maximum(n, 1.0))).reshape(-1)",
       "return (mb / max(mb.sum(), 1.0)).reshape(-1)")]),
    ("sequence mean: the 1 / B dropped",
     [("return (mb / (mb.shape[0] * np.maximum(n, 1.0))).reshape(-1)",
       "return (mb / np.maximum(n, 1.0)).reshape(-1)")]),
    ("sequence mean: empty completions left out of B",
     [("return (mb / (mb.shape[0] * np.maximum(n, 1.0))).reshape(-1)",
       "return (mb / (max(int((n > 0).sum()), 1) * np.maximum(n, 1.0))).reshape(-1)")]),
    ("fp8 decode: exponent bias 8",
     [("(1.0 + m / 8.0) * np.exp2(e - 7.0)", "(1.0 + m / 8.0) * np.exp2(e - 8.0)")]),
    ("fp8 decode: subnormals on the normal scale",
     [("np.where(e == 0, m / 8.0 * 2.0 ** -6,", "np.where(e == 0, m / 8.0 * 2.0 ** -7,")]),
    ("fp8 encode: ties away from zero",
     [("np.where(codes[lo] % 2 == 0, lo, hi)", "hi")]),
    ("fp8 encode: sign dropped",
     [("out = np.where(neg, out | 0x80, out).astype(np.uint8)", "out = out.astype(np.uint8)")]),
    ("fp8 scale: one binade too large",
     [("return int(k - 9) if f <= 0.875 else int(k - 8)", "return int(k - 8)")]),
    ("fp8 quantize: tensor scale from the first row",
     [("e = np.array([fp8_scale_exponent(np.abs(X).max() if X.size else 0.0)])",
       "e = np.array([fp8_scale_exponent(np.abs(X[0]).max() if X.size else 0.0)])")]),
    ("backward: recomputed logits against the transposed head",
     [("Z = Hs @ Wf.T", "Z = Hs @ Wf[::-1].T")]),
    ("backward: dW overwritten by each row block",
     [("dW += dZ.T @ Hs", "dW = dZ.T @ Hs")]),
    ("backward: row blocks past the first skipped",
     [("sel = need[b0:b0 + block]", "sel = need[b0:block]")]),
    ("backward: only the requested dH rows visited (unmasked tokens not added)",
     [("need = np.union1d(active, rows) if want_dW else np.unique(rows)",
       "need = np.unique(rows)")]),
]


def _load(edits):
    src = open(SOURCE_PATH).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("grpo_oracle_mutant")
    mod.__file__ = SOURCE_PATH
    exec(compile(src, "grpo_oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pin_cases():
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            yield name, fn, {}
            continue
        argnames, values = marks[0].args[0], marks[0].args[1]
        names = [a.strip() for a in argnames.split(",")]
        for v in values:
            yield f"{name}{v}", fn, dict(zip(names, v if len(names) > 1 else [v]))


def _failing_pins(mod, monkeypatch):
    for n in PUBLIC:
        monkeypatch.setattr(oracle, n, getattr(mod, n))
        monkeypatch.setattr(grpo_oracle, n, getattr(mod, n))
    failed = []
    for name, fn, kw in _pin_cases():
        try:
            fn(**kw)
        except Exception:       # an assertion, or the mutant breaking outright
            failed.append(name)
    monkeypatch.undo()
    return failed


def test_unmutated_source_passes_every_pin(monkeypatch):
    assert _failing_pins(_load([]), monkeypatch) == []


@pytest.mark.parametrize("name,edits", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, edits, monkeypatch):
    failed = _failing_pins(_load(edits), monkeypatch)
    assert failed, f"no pin catches: {name}"
