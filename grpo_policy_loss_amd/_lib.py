"""ctypes binding of libgrpo.so (include/grpo.h).

Argument marshalling only: every step of the loss runs in the HIP library.
torch supplies device memory (outputs and workspace) and the current stream.
There is no CPU fallback: without the built library or a GPU every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgrpo.so")

GRPO_F32, GRPO_BF16, GRPO_FP8_E4M3 = 0, 1, 2
GRPO_OP_REF, GRPO_OP_FWD, GRPO_OP_BWD, GRPO_OP_BWD_MIN = 0, 1, 2, 3
STATUS = {0: "GRPO_OK", -1: "GRPO_ERR_INVALID_ARG", -2: "GRPO_ERR_WORKSPACE",
          -3: "GRPO_ERR_UNSUPPORTED", -4: "GRPO_ERR_HIP"}

_i64, _f32, _vp, _sz, _int = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int



class Opts(ctypes.Structure):
    """grpo_opts: zero fields give the plain loss (temperature 0 means 1)."""
    _fields_ = [("logit_scale_multiply", ctypes.c_float), ("logit_scale_divide", ctypes.c_float),
                ("logit_softcapping", ctypes.c_float), ("temperature", ctypes.c_float),
                ("kl_estimator", ctypes.c_int32), ("no_detach", ctypes.c_int32),
                ("aggregation", ctypes.c_int32)]


# grpo_kl_estimator and grpo_aggregation
KL_REVERSE, KL_FORWARD, KL_REVERSE_Q = 0, 1, 2
AGG_TOKEN_MEAN, AGG_SEQUENCE_MEAN = 0, 1


_OPTS_P = ctypes.POINTER(Opts)

# name -> (restype, argtypes); mirrors include/grpo.h
SIGNATURES = {
    "grpo_workspace_bytes": (_sz, [_int, _i64, _i64, _i64, _int, _i64]),
    "grpo_advantages": (_int, [_vp, _i64, _i64, _f32, _vp, _vp]),
    "grpo_ref_logprobs": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _i64, _vp, _vp, _sz, _vp]),
    "grpo_loss_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _f32,
                             _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "grpo_loss_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int,
                             _f32, _f32, _i64, _vp, _vp, _vp, _sz, _vp]),
    "grpo_ref_logprobs_ex": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _i64, _OPTS_P, _vp,
                                    _vp, _sz, _vp]),
    "grpo_loss_fwd_ex": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _f32,
                                _i64, _OPTS_P, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "grpo_loss_bwd_ex": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                _int, _f32, _f32, _i64, _OPTS_P, _vp, _vp, _vp, _sz, _vp]),
    "grpo_gemm_nt": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _vp, _vp]),
    "grpo_noalloc_scratch_bytes": (_sz, []),
    "grpo_loss_fwd_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int,
                                     _f32, _i64, _OPTS_P, _vp, _vp, _vp, _vp, _vp]),
    "grpo_auto_chunk": (_i64, [_i64, _i64, _i64, _i64, _int, _sz]),
    "grpo_quantize_fp8_workspace_bytes": (_sz, []),
    "grpo_quantize_fp8": (_int, [_vp, _int, _i64, _i64, _int, _vp, _vp, _vp, _sz, _vp]),
    "grpo_dequantize_fp8": (_int, [_vp, _vp, _i64, _i64, _int, _vp, _vp]),
    "grpo_ref_logprobs_fp8": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _OPTS_P,
                                     _vp, _vp, _sz, _vp]),
    "grpo_loss_fwd_fp8": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                 _f32, _i64, _OPTS_P, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "grpo_loss_bwd_fp8": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                 _i64, _i64, _f32, _f32, _i64, _OPTS_P, _vp, _vp, _vp, _sz, _vp]),
    "grpo_timing_begin": (_int, []),
    "grpo_timing_end": (_int, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_int),
                               ctypes.POINTER(ctypes.c_double), _int]),
    "grpo_strerror": (ctypes.c_char_p, [_int]),
    "grpo_last_error": (ctypes.c_char_p, []),
}


class GrpoError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}: {detail}")
        self.code = code


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libgrpo.so (built in-tree by grpo_policy_loss_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with grpo_policy_loss_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(fn: str, code: int):
    if code != 0:
        raise GrpoError(fn, code, lib().grpo_last_error().decode(errors="replace"))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GRPO_F32
    if t.dtype == torch.bfloat16:
        return GRPO_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _arg(t, name, dtype=None, shape=None, numel=None):
    """Check one tensor argument's type, dtype and size before any device call.
    The C ABI cannot see buffer sizes, so this is the only guard against a
    kernel writing past an output or reading past an input."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t


def _matrix(t, name):
    _arg(t, name)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _opts(opts):
    """A grpo_opts pointer from a dict of its fields (None: the plain loss)."""
    if opts is None:
        return None
    kinds = dict(Opts._fields_)
    unknown = set(opts) - set(kinds)
    if unknown:
        raise ValueError(f"unknown options: {sorted(unknown)}")
    return ctypes.pointer(Opts(**{k: (float(v) if kinds[k] is ctypes.c_float else int(v))
                                  for k, v in opts.items()}))


def grpo_workspace_bytes(op: int, N: int, d: int, V: int, dtype: int, chunk: int) -> int:
    return int(lib().grpo_workspace_bytes(op, N, d, V, dtype, chunk))


def auto_chunk(B: int, L: int, d: int, V: int, dtype: int, budget_bytes=None) -> int:
    """grpo_auto_chunk: tokens per chunk for B sequences of L tokens.  budget_bytes
    None: half of the current device's free HBM (torch.cuda.mem_get_info)."""
    if budget_bytes is None:
        budget_bytes = torch.cuda.mem_get_info()[0] // 2
    c = int(lib().grpo_auto_chunk(B, L, d, V, dtype, int(budget_bytes)))
    if c <= 0:
        _check("grpo_auto_chunk", -1)
    return c


def _check_workspace(workspace, op, N, d, V, dt, chunk):
    """A caller's workspace must be a uint8 tensor of at least the op's minimum size
    (the backward plans its dZ slab from the size it is given)."""
    if workspace is None:
        return
    _arg(workspace, "workspace", dtype=torch.uint8)
    if chunk == 0:
        return                      # checked again once the chunk is known
    least = grpo_workspace_bytes(GRPO_OP_BWD_MIN if op == GRPO_OP_BWD else op, N, d, V, dt, chunk)
    if least == 0:
        _check("grpo_workspace_bytes", -1)
    if workspace.numel() < least:
        raise ValueError(f"workspace holds {workspace.numel()} bytes; this call needs at least {least}")


def _workspace(op, N, d, V, dt, chunk, device, workspace):
    """The caller's workspace, or a new one of grpo_workspace_bytes(op, ...) bytes."""
    if workspace is not None:
        _check_workspace(workspace, op, N, d, V, dt, chunk)
        _dev(workspace)
        return workspace
    need = grpo_workspace_bytes(op, N, d, V, dt, chunk)
    if need == 0:
        _check("grpo_workspace_bytes", -1)
    return torch.empty(need, dtype=torch.uint8, device=device)


def grpo_advantages(rewards: torch.Tensor, group_size: int, eps: float = 1e-4, out=None):
    _arg(rewards, "rewards", dtype=torch.float32)
    if group_size <= 0 or rewards.numel() % group_size:
        raise ValueError("rewards length must be a positive multiple of group_size")
    out = torch.empty_like(rewards) if out is None else \
        _arg(out, "out", dtype=torch.float32, numel=rewards.numel())
    _dev(rewards, out)
    _check("grpo_advantages", lib().grpo_advantages(
        _ptr(rewards), rewards.numel() // group_size, group_size, eps, _ptr(out), _stream()))
    return out


def grpo_ref_logprobs(H_ref, W, y, chunk: int = 4096, out=None, workspace=None,
                      opts=None):
    N, d = _matrix(H_ref, "H_ref")
    dt = _dt(H_ref)
    V = _matrix(W, "W")[0]
    _arg(W, "W", dtype=H_ref.dtype, shape=(V, d))
    _arg(y, "y", dtype=torch.int32, numel=N)
    out = torch.empty(N, dtype=torch.float32, device=H_ref.device) if out is None else \
        _arg(out, "out", dtype=torch.float32, numel=N)
    _check_workspace(workspace, GRPO_OP_REF, N, d, V, dt, chunk)
    _dev(H_ref, W, y, out)
    if chunk == 0:
        chunk = auto_chunk(1, N, d, V, dt)
    ws = _workspace(GRPO_OP_REF, N, d, V, dt, chunk, H_ref.device, workspace)
    _check("grpo_ref_logprobs_ex", lib().grpo_ref_logprobs_ex(
        _ptr(H_ref), _ptr(W), _ptr(y), N, d, V, dt, chunk, _opts(opts), _ptr(out), _ptr(ws),
        ws.numel(), _stream()))
    return out


def grpo_loss_fwd(H, W, y, mask, adv, ref_lp, B: int, L: int, beta: float = 0.04,
                  chunk: int = 4096, workspace=None, opts=None):
    """Returns (loss[1], lp[N], kl[N], lse[N]), all float32 on the GPU.  `opts`: dict
    of grpo_opts fields (logit_scale_multiply, logit_scale_divide, logit_softcapping,
    temperature, kl_estimator, no_detach, aggregation), or None for the plain loss.
    chunk 0 (here and in the other calls): auto_chunk with half the free HBM."""
    N, d = _matrix(H, "H")
    dt = _dt(H)
    V = _matrix(W, "W")[0]
    _arg(W, "W", dtype=H.dtype, shape=(V, d))
    if N != B * L:
        raise ValueError(f"H has {N} rows, B * L = {B * L}")
    _arg(y, "y", dtype=torch.int32, numel=N)
    _arg(mask, "mask", dtype=torch.uint8, numel=N)
    _arg(adv, "adv", dtype=torch.float32, numel=B)
    _arg(ref_lp, "ref_lp", dtype=torch.float32, numel=N)
    _check_workspace(workspace, GRPO_OP_FWD, N, d, V, dt, chunk)
    _dev(H, W, y, mask, adv, ref_lp)
    dev = H.device
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lp = torch.empty(N, dtype=torch.float32, device=dev)
    kl = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    if chunk == 0:
        chunk = auto_chunk(B, L, d, V, dt)
    ws = _workspace(GRPO_OP_FWD, N, d, V, dt, chunk, dev, workspace)
    _check("grpo_loss_fwd_ex", lib().grpo_loss_fwd_ex(
        _ptr(H), _ptr(W), _ptr(y), _ptr(mask), _ptr(adv), _ptr(ref_lp), B, L, d, V, dt, beta,
        chunk, _opts(opts), _ptr(loss), _ptr(lp), _ptr(kl), _ptr(lse), _ptr(ws),
        ws.numel(), _stream()))
    return loss, lp, kl, lse


def grpo_loss_bwd(H, W, y, mask, adv, ref_lp, lp, lse, B: int, L: int, beta: float = 0.04,
                  grad_loss: float = 1.0, chunk: int = 4096, dW=None, dH=None, workspace=None,
                  opts=None):
    """Returns (dH[N, d] in H's dtype, dW[V, d] float32).  dW is accumulated into
    when given (zeros are allocated otherwise).  `opts` must be those of the
    forward that produced lp and lse."""
    N, d = _matrix(H, "H")
    dt = _dt(H)
    V = _matrix(W, "W")[0]
    _arg(W, "W", dtype=H.dtype, shape=(V, d))
    if N != B * L:
        raise ValueError(f"H has {N} rows, B * L = {B * L}")
    _arg(y, "y", dtype=torch.int32, numel=N)
    _arg(mask, "mask", dtype=torch.uint8, numel=N)
    _arg(adv, "adv", dtype=torch.float32, numel=B)
    for t, name in ((ref_lp, "ref_lp"), (lp, "lp"), (lse, "lse")):
        _arg(t, name, dtype=torch.float32, numel=N)
    dev = H.device
    dH = torch.empty_like(H) if dH is None else _arg(dH, "dH", dtype=H.dtype, shape=(N, d))
    dW = torch.zeros(V, d, dtype=torch.float32, device=dev) if dW is None else \
        _arg(dW, "dW", dtype=torch.float32, shape=(V, d))
    _check_workspace(workspace, GRPO_OP_BWD, N, d, V, dt, chunk)
    _dev(H, W, y, mask, adv, ref_lp, lp, lse, dH, dW)
    if chunk == 0:
        chunk = auto_chunk(B, L, d, V, dt)
    ws = _workspace(GRPO_OP_BWD, N, d, V, dt, chunk, dev, workspace)
    _check("grpo_loss_bwd_ex", lib().grpo_loss_bwd_ex(
        _ptr(H), _ptr(W), _ptr(y), _ptr(mask), _ptr(adv), _ptr(ref_lp), _ptr(lp), _ptr(lse),
        B, L, d, V, dt, beta, grad_loss, chunk, _opts(opts), _ptr(dH), _ptr(dW), _ptr(ws),
        ws.numel(), _stream()))
    return dH, dW


def grpo_timing_begin():
    """Start per-kernel HIP-event timing of this thread's library launches."""
    lib().grpo_timing_begin()


def grpo_timing_end(max_entries: int = 32):
    """Stop timing; {kernel name: (launches, total milliseconds)}."""
    names = (ctypes.c_char_p * max_entries)()
    launches = (_int * max_entries)()
    ms = (ctypes.c_double * max_entries)()
    n = lib().grpo_timing_end(names, launches, ms, max_entries)
    return {names[i].decode(): (launches[i], ms[i]) for i in range(min(n, max_entries))}


def grpo_gemm_nt(A, B):
    """C = A @ B.T in float32 through the library's MFMA tile main loop."""
    M, K = _matrix(A, "A")
    _dt(A)
    N = _matrix(B, "B")[0]
    _arg(B, "B", dtype=A.dtype, shape=(N, K))
    _dev(A, B)
    C = torch.empty(M, N, dtype=torch.float32, device=A.device)
    _check("grpo_gemm_nt", lib().grpo_gemm_nt(_ptr(A), _ptr(B), M, N, K, _dt(A), _ptr(C), _stream()))
    return C


# ---------------------------------------------------------------- fp8 e4m3 path
class Fp8:
    """Float8 e4m3 codes (uint8, [rows, cols]) and their power-of-two scales
    (float32 on the GPU: one per row, or one for the tensor)."""

    def __init__(self, codes, scales, per_row):
        self.codes, self.scales, self.per_row = codes, scales, per_row

    @property
    def shape(self):
        return self.codes.shape


def quantize_fp8(X, per_row=True) -> Fp8:
    """grpo_quantize_fp8 of a float32 or bfloat16 matrix on the GPU."""
    rows, cols = _matrix(X, "X")
    _dt(X)
    _dev(X)
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=X.device)
    scales = torch.empty(rows if per_row else 1, dtype=torch.float32, device=X.device)
    ws = None if per_row else torch.empty(int(lib().grpo_quantize_fp8_workspace_bytes()),
                                          dtype=torch.uint8, device=X.device)
    _check("grpo_quantize_fp8", lib().grpo_quantize_fp8(
        _ptr(X), _dt(X), rows, cols, int(per_row), _ptr(codes), _ptr(scales), _ptr(ws),
        0 if ws is None else ws.numel(), _stream()))
    return Fp8(codes, scales, per_row)


def dequantize_fp8(q: Fp8):
    """grpo_dequantize_fp8: the exact bfloat16 values of q."""
    rows, cols = _matrix(q.codes, "codes")
    _arg(q.codes, "codes", dtype=torch.uint8)
    _arg(q.scales, "scales", dtype=torch.float32, numel=rows if q.per_row else 1)
    _dev(q.codes, q.scales)
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device=q.codes.device)
    _check("grpo_dequantize_fp8", lib().grpo_dequantize_fp8(
        _ptr(q.codes), _ptr(q.scales), rows, cols, int(q.per_row), _ptr(out), _stream()))
    return out


def _fp8_args(H: Fp8, W: Fp8):
    if not H.per_row or W.per_row:
        raise ValueError("fp8 loss takes per-row H scales and one W scale")
    N, d = _matrix(H.codes, "H codes")
    V = _matrix(W.codes, "W codes")[0]
    _arg(H.codes, "H codes", dtype=torch.uint8)
    _arg(W.codes, "W codes", dtype=torch.uint8, shape=(V, d))
    _arg(H.scales, "H scales", dtype=torch.float32, numel=N)
    _arg(W.scales, "W scales", dtype=torch.float32, numel=1)
    return N, d, V


def grpo_ref_logprobs_fp8(H_ref: Fp8, W: Fp8, y, chunk: int = 4096, out=None, workspace=None,
                          opts=None):
    N, d, V = _fp8_args(H_ref, W)
    _arg(y, "y", dtype=torch.int32, numel=N)
    out = torch.empty(N, dtype=torch.float32, device=y.device) if out is None else \
        _arg(out, "out", dtype=torch.float32, numel=N)
    _check_workspace(workspace, GRPO_OP_REF, N, d, V, GRPO_FP8_E4M3, chunk)
    _dev(H_ref.codes, H_ref.scales, W.codes, W.scales, y, out)
    if chunk == 0:
        chunk = auto_chunk(1, N, d, V, GRPO_FP8_E4M3)
    ws = _workspace(GRPO_OP_REF, N, d, V, GRPO_FP8_E4M3, chunk, y.device, workspace)
    _check("grpo_ref_logprobs_fp8", lib().grpo_ref_logprobs_fp8(
        _ptr(H_ref.codes), _ptr(H_ref.scales), _ptr(W.codes), _ptr(W.scales), _ptr(y), N, d, V,
        chunk, _opts(opts), _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def grpo_loss_fwd_fp8(H: Fp8, W: Fp8, y, mask, adv, ref_lp, B: int, L: int, beta: float = 0.04,
                      chunk: int = 4096, workspace=None, opts=None):
    """grpo_loss_fwd on fp8 operands: (loss[1], lp[N], kl[N], lse[N])."""
    N, d, V = _fp8_args(H, W)
    if N != B * L:
        raise ValueError(f"H has {N} rows, B * L = {B * L}")
    _arg(y, "y", dtype=torch.int32, numel=N)
    _arg(mask, "mask", dtype=torch.uint8, numel=N)
    _arg(adv, "adv", dtype=torch.float32, numel=B)
    _arg(ref_lp, "ref_lp", dtype=torch.float32, numel=N)
    _check_workspace(workspace, GRPO_OP_FWD, N, d, V, GRPO_FP8_E4M3, chunk)
    _dev(H.codes, H.scales, W.codes, W.scales, y, mask, adv, ref_lp)
    dev = y.device
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lp, kl, lse = (torch.empty(N, dtype=torch.float32, device=dev) for _ in range(3))
    if chunk == 0:
        chunk = auto_chunk(B, L, d, V, GRPO_FP8_E4M3)
    ws = _workspace(GRPO_OP_FWD, N, d, V, GRPO_FP8_E4M3, chunk, dev, workspace)
    _check("grpo_loss_fwd_fp8", lib().grpo_loss_fwd_fp8(
        _ptr(H.codes), _ptr(H.scales), _ptr(W.codes), _ptr(W.scales), _ptr(y), _ptr(mask),
        _ptr(adv), _ptr(ref_lp), B, L, d, V, beta, chunk, _opts(opts), _ptr(loss), _ptr(lp),
        _ptr(kl), _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return loss, lp, kl, lse


def grpo_loss_bwd_fp8(H: Fp8, W: Fp8, y, mask, adv, ref_lp, lp, lse, B: int, L: int,
                      beta: float = 0.04, grad_loss: float = 1.0, chunk: int = 4096, dW=None,
                      dH=None, workspace=None, opts=None):
    """Backward of grpo_loss_fwd_fp8 with respect to the dequantised H and W:
    (dH[N, d] bfloat16, dW[V, d] float32, accumulated into when given)."""
    N, d, V = _fp8_args(H, W)
    if N != B * L:
        raise ValueError(f"H has {N} rows, B * L = {B * L}")
    _arg(y, "y", dtype=torch.int32, numel=N)
    _arg(mask, "mask", dtype=torch.uint8, numel=N)
    _arg(adv, "adv", dtype=torch.float32, numel=B)
    for t, name in ((ref_lp, "ref_lp"), (lp, "lp"), (lse, "lse")):
        _arg(t, name, dtype=torch.float32, numel=N)
    dev = y.device
    dH = torch.empty(N, d, dtype=torch.bfloat16, device=dev) if dH is None else \
        _arg(dH, "dH", dtype=torch.bfloat16, shape=(N, d))
    dW = torch.zeros(V, d, dtype=torch.float32, device=dev) if dW is None else \
        _arg(dW, "dW", dtype=torch.float32, shape=(V, d))
    _check_workspace(workspace, GRPO_OP_BWD, N, d, V, GRPO_FP8_E4M3, chunk)
    _dev(H.codes, H.scales, W.codes, W.scales, y, mask, adv, ref_lp, lp, lse, dH, dW)
    if chunk == 0:
        chunk = auto_chunk(B, L, d, V, GRPO_FP8_E4M3)
    ws = _workspace(GRPO_OP_BWD, N, d, V, GRPO_FP8_E4M3, chunk, dev, workspace)
    _check("grpo_loss_bwd_fp8", lib().grpo_loss_bwd_fp8(
        _ptr(H.codes), _ptr(H.scales), _ptr(W.codes), _ptr(W.scales), _ptr(y), _ptr(mask),
        _ptr(adv), _ptr(ref_lp), _ptr(lp), _ptr(lse), B, L, d, V, beta, grad_loss, chunk,
        _opts(opts), _ptr(dH), _ptr(dW), _ptr(ws), ws.numel(), _stream()))
    return dH, dW
