"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/grpo.h declares, sizes workspaces sanely, and rejects bad
arguments on the host before anything is enqueued (no compute call is made
with valid arguments here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grpo.h")

gp = pytest.importorskip("grpo_policy_loss_amd")
from grpo_policy_loss_amd import _lib  # noqa: E402

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libgrpo.so not built", allow_module_level=True)

L = _lib.lib()
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(grpo_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_four_calls_and_helpers():
    names = declared_functions()
    for n in ["grpo_advantages", "grpo_ref_logprobs", "grpo_loss_fwd", "grpo_loss_bwd",
              "grpo_workspace_bytes", "grpo_strerror", "grpo_last_error", "grpo_gemm_nt"]:
        assert n in names, names


def test_library_exports_every_declared_symbol():
    for n in declared_functions():
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, f"binding lacks a signature for {n}"


def test_strerror_texts():
    for code in [0, -1, -2, -3, -4, 7]:
        assert L.grpo_strerror(code)


@pytest.mark.parametrize("op", [0, 1, 2, 3])
def test_workspace_bytes_bounded_and_independent_of_N_times_V(op):
    # long-context shape: 163840 tokens, V 128256, d 4096, chunk 8192
    N, d, V, chunk = 163840, 4096, 128256, 8192
    ws = L.grpo_workspace_bytes(op, N, d, V, 1, chunk)
    assert ws > 0
    assert ws < N * V * 4 / 10           # far below the float32 (tokens x vocab) logits
    if op >= 2:
        # one dZ slab (at most the whole padded vocabulary of one chunk, bf16), the
        # chunk's hidden states and their transpose, dH split partials (at most 8
        # float32 copies of a chunk) and 8 B per token (index list, counts); no
        # copy of W and no second slab
        Vp = -(-V // 256) * 256
        assert ws <= chunk * Vp * 2 + 2 * chunk * d * 2 + 8 * chunk * d * 4 + 8 * N + (1 << 20)
        # grows with N only through the index list and the counts (8 B per token)
        ws2 = L.grpo_workspace_bytes(op, 2 * N, d, V, 1, chunk)
        assert ws2 - ws <= 8 * N + 1024
    if op == 2:
        # the default slab budget, 1.25 GiB: 81920 of the 128256 vocabulary columns
        # of an 8192-token chunk (two slabs per chunk)
        least = L.grpo_workspace_bytes(3, N, d, V, 1, chunk)
        assert ws - least == chunk * (81920 - 256) * 2


def test_backward_workspace_plans_the_slab_from_its_size():
    # Qwen2.5-1.5B shape, bf16: the default holds the whole vocabulary in one slab
    # (4096 x 151936 x 2 B = 1.16 GiB, within the 1.25 GiB budget); the minimum
    # holds one 256-column slab
    N, d, V, chunk = 32768, 1536, 151936, 4096
    full = L.grpo_workspace_bytes(2, N, d, V, 1, chunk)
    least = L.grpo_workspace_bytes(3, N, d, V, 1, chunk)
    Vp = -(-V // 256) * 256
    assert full - least == chunk * (Vp - 256) * 2
    # below the minimum: refused on the host before any launch
    one = ctypes.c_void_p(16)
    def bwd(wsb):
        return L.grpo_loss_bwd(one, one, one, one, one, one, one, one, 32, 1024, d, V, 1, 0.04,
                               1.0, chunk, one, one, one, wsb, None)
    assert bwd(least - 1) == -2
    assert b"at least" in L.grpo_last_error()
    # f32 and fp8 plans too
    assert L.grpo_workspace_bytes(3, 512, 256, 1024, 0, 128) < L.grpo_workspace_bytes(2, 512, 256, 1024, 0, 128)
    assert L.grpo_workspace_bytes(3, N, d, V, 2, chunk) < L.grpo_workspace_bytes(2, N, d, V, 2, chunk)


def test_slab_stays_inside_one_buffer_resource():
    # a 16384-token chunk at d 4096: 16384 x 128256 x 2 B would pass 2^31, so the
    # default plan narrows the slab (the dW GEMM reads it through one resource)
    N, d, V, chunk = 163840, 4096, 128256, 16384
    ws = L.grpo_workspace_bytes(2, N, d, V, 1, chunk)
    fixed = L.grpo_workspace_bytes(3, N, d, V, 1, chunk) - chunk * 256 * 2
    assert (ws - fixed) < (1 << 31)
    # asking for more memory does not widen it past the bound either: the call
    # accepts a huge workspace and plans within the bound (checked by the GPU tests)
    assert L.grpo_workspace_bytes(2, N, d, V, 1, chunk) == ws


def test_environment_does_not_change_the_plan(monkeypatch):
    N, d, V, chunk = 32768, 1536, 151936, 4096
    a = L.grpo_workspace_bytes(2, N, d, V, 1, chunk)
    monkeypatch.setenv("GRPO_SLAB_MIB", "256")
    assert L.grpo_workspace_bytes(2, N, d, V, 1, chunk) == a


def test_workspace_bytes_rejects_bad_shapes():
    assert L.grpo_workspace_bytes(1, 0, 256, 1024, 0, 128) == 0
    assert L.grpo_workspace_bytes(1, 512, 255, 1024, 0, 128) == 0      # d not multiple of 4
    assert L.grpo_workspace_bytes(1, 512, 260, 1024, 1, 128) == 0      # bf16 needs multiple of 8
    assert L.grpo_workspace_bytes(1, 512, 256, 1024, 5, 128) == 0      # bad dtype
    assert L.grpo_workspace_bytes(9, 512, 256, 1024, 0, 128) == 0      # bad op
    assert L.grpo_workspace_bytes(-1, 512, 256, 1024, 0, 128) == 0


def _fwd(**kw):
    a = dict(H=FAKE, W=FAKE, y=FAKE, mask=FAKE, adv=FAKE, ref=FAKE, B=8, L=64, d=256, V=1024,
             dt=0, beta=0.04, chunk=128, loss=FAKE, lp=FAKE, kl=FAKE, lse=FAKE, ws=FAKE,
             wsb=1 << 40, s=None)
    a.update(kw)
    return L.grpo_loss_fwd(a["H"], a["W"], a["y"], a["mask"], a["adv"], a["ref"], a["B"], a["L"],
                           a["d"], a["V"], a["dt"], a["beta"], a["chunk"], a["loss"], a["lp"],
                           a["kl"], a["lse"], a["ws"], a["wsb"], a["s"])


def test_loss_fwd_argument_errors():
    assert _fwd(H=None) == -1
    assert _fwd(lse=None) == -1
    assert _fwd(B=0) == -1
    assert _fwd(d=-4) == -1
    assert _fwd(dt=3) == -1
    assert _fwd(beta=float("nan")) == -1
    assert _fwd(beta=float("inf")) == -1
    assert _fwd(d=250) == -3
    assert _fwd(ws=None) == -2
    assert _fwd(wsb=16) == -2
    assert b"workspace" in L.grpo_last_error()


def test_loss_bwd_argument_errors():
    def bwd(**kw):
        a = dict(H=FAKE, dH=FAKE, dW=FAKE, g=1.0, wsb=1 << 40, ws=FAKE, B=8)
        a.update(kw)
        return L.grpo_loss_bwd(a["H"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], 64, 256,
                               1024, 0, 0.04, a["g"], 128, a["dH"], a["dW"], a["ws"], a["wsb"],
                               None)
    assert bwd(dW=None) == -1
    assert bwd(dH=None) == -1
    assert bwd(g=float("nan")) == -1
    assert bwd(B=-1) == -1
    assert bwd(wsb=0) == -2


def test_ref_and_advantages_argument_errors():
    assert L.grpo_ref_logprobs(FAKE, FAKE, None, 512, 256, 1024, 0, 128, FAKE, FAKE, 1 << 40, None) == -1
    assert L.grpo_ref_logprobs(FAKE, FAKE, FAKE, 512, 256, 1024, 0, 0, FAKE, FAKE, 1 << 40, None) == -1
    assert L.grpo_ref_logprobs(FAKE, FAKE, FAKE, 512, 256, 1024, 0, 128, FAKE, FAKE, 8, None) == -2
    assert L.grpo_advantages(None, 2, 4, 1e-4, FAKE, None) == -1
    assert L.grpo_advantages(FAKE, 0, 4, 1e-4, FAKE, None) == -1
    assert L.grpo_advantages(FAKE, 2, 4, float("nan"), FAKE, None) == -1
    assert L.grpo_gemm_nt(FAKE, FAKE, 4, 4, 6, 1, FAKE, None) == -3    # 12 B rows


def test_binding_refuses_cpu_tensors():
    import torch
    H = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        gp.grpo_ref_logprobs(H, torch.zeros(16, 8), torch.zeros(4, dtype=torch.int32))


@pytest.mark.parametrize("field,value,msg", [
    ("temperature", -1.0, b"logit opts"), ("logit_softcapping", -30.0, b"logit opts"),
    ("logit_scale_multiply", float("nan"), b"logit opts"),
    ("logit_scale_divide", float("inf"), b"logit opts"),
    ("kl_estimator", 3, b"kl_estimator"), ("kl_estimator", -1, b"kl_estimator"),
    ("no_detach", 2, b"no_detach"), ("aggregation", 2, b"aggregation")])
def test_opts_rejected_before_any_launch(field, value, msg):
    import ctypes
    opts = _lib.Opts(**{field: value})
    one = ctypes.c_void_p(16)        # never dereferenced: the options are checked first
    st = L.grpo_ref_logprobs_ex(one, one, one, 8, 16, 32, 0, 8, ctypes.pointer(opts), one, one,
                                1 << 20, None)
    assert st == -1
    assert msg in L.grpo_last_error()
    st = L.grpo_loss_fwd_ex(one, one, one, one, one, one, 2, 4, 16, 32, 0, 0.04, 8,
                            ctypes.pointer(opts), one, one, one, one, one, 1 << 20, None)
    assert st == -1
    st = L.grpo_loss_bwd_ex(one, one, one, one, one, one, one, one, 2, 4, 16, 32, 0, 0.04, 1.0, 8,
                            ctypes.pointer(opts), one, one, one, 1 << 20, None)
    assert st == -1


def test_opts_struct_matches_the_header():
    """Field order and types of grpo_opts as the header declares them."""
    import ctypes
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "grpo.h")).read()
    body = hdr[hdr.index("typedef struct grpo_opts {"):hdr.index("} grpo_opts;")]
    decl = [ln.split(";")[0].split() for ln in body.splitlines()[1:] if ";" in ln]
    want = [(name, {"float": ctypes.c_float, "int32_t": ctypes.c_int32}[ty]) for ty, name in decl]
    assert list(_lib.Opts._fields_) == want


def test_auto_chunk_is_the_largest_fitting_multiple_of_256():
    """grpo_auto_chunk (pure host arithmetic): a multiple of 256 up to 8192 and up to N,
    whose forward + backward workspace fits the budget, and the largest such."""
    def ws(N, d, V, c):
        return L.grpo_workspace_bytes(1, N, d, V, 1, c) + L.grpo_workspace_bytes(2, N, d, V, 1, c)
    for (B, Lq, d, V) in [(32, 1024, 1536, 151936), (8, 4096, 4096, 128256),
                          (8, 20480, 4096, 128256), (4, 16384, 2880, 201088)]:
        N = B * Lq
        # unlimited memory: the speed cap
        assert L.grpo_auto_chunk(B, Lq, d, V, 1, 1 << 62) == 8192
        for budget in (ws(N, d, V, 256) + 1, ws(N, d, V, 3000), ws(N, d, V, 8192) - 1, 12 << 30):
            c = L.grpo_auto_chunk(B, Lq, d, V, 1, budget)
            assert c % 256 == 0 and 256 <= c <= 8192
            assert ws(N, d, V, c) <= budget
            if c < 8192:
                assert ws(N, d, V, c + 256) > budget
    # nothing fits: the smallest candidate
    assert L.grpo_auto_chunk(32, 1024, 1536, 151936, 1, 1024) == 256
    # short inputs: capped at N rounded up to 256
    assert L.grpo_auto_chunk(3, 100, 64, 500, 0, 1 << 62) == 512
    assert L.grpo_auto_chunk(1, 7, 16, 3, 0, 1 << 62) == 256
    # invalid arguments
    assert L.grpo_auto_chunk(0, 8, 16, 32, 1, 1 << 30) == 0
    assert L.grpo_auto_chunk(2, 8, 16, 32, 7, 1 << 30) == 0
    assert L.grpo_auto_chunk(2, 8, 0, 32, 1, 1 << 30) == 0
