"""exact_tiled_attention_fa_amd: exact tiled (FlashAttention-style) attention on MI355X.

Thin Python binding over the C ABI in include/fa.h (libfa.so, hand-written HIP
kernels for gfx950). torch supplies device memory and the current stream
only; every step of the computation runs in the library's kernels.

    o, lse = fwd(q, k, v, causal=False, scale=None)
    o = attention(q, k, v, causal=False, scale=None)     # differentiable
    o, lse = fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal=False, scale=None)
    o, lse = decode(q, k, v, num_splits=16, scale=None)
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import FaError

__all__ = ["attention", "fwd", "fwd_noalloc", "fwd_fp8", "decode", "bwd", "fwd_workspace_bytes", "decode_workspace_bytes",
           "bwd_workspace_bytes", "prepare_fwd", "prepare_fwd_fp8", "prepare_decode", "prepare_bwd",
           "FaError"]


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _one_device(*named) -> torch.device:
    """The one GPU that every given tensor lives on: the kernels run there and
    read or write all of them, so a tensor elsewhere (another GPU, host
    memory) is refused before any launch. None entries are skipped."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device (got {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device} but the other tensors are on {dev}: all must share one GPU")
    return dev


def _check_bf16(name: str, t: torch.Tensor, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16 (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: float | None = None, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None):
    """Attention forward. q [B,Hq,N,d], k/v [B,Hkv,N,d] bf16 -> (o [B,Hq,N,d] bf16, lse [B,Hq,N] fp32)."""
    return _fwd_call("fa_fwd", q, k, v, causal, scale, out, lse)


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                causal: bool = False, scale: float | None = None):
    """fwd through fa_fwd_noalloc: the library allocates nothing (key-split
    partials in its static per-GPU scratch), and the caller passes out and lse.
    Calls that may overlap on one GPU must be ordered by the caller."""
    if out is None or lse is None:
        raise ValueError("fwd_noalloc writes into caller-provided out and lse")
    return _fwd_call("fa_fwd_noalloc", q, k, v, causal, scale, out, lse)


def _fwd_call(entry: str, q, k, v, causal, scale, out, lse):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t, 4)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError(f"k and v must be [B,Hkv,N,d] = {(B, Hkv, N, d)}; got {tuple(k.shape)}, {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_bf16("out", out, 4)
    if out.shape != q.shape:
        raise ValueError("out must match q's shape")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,Hq,N] tensor")
    dev = _one_device(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse))
    with torch.cuda.device(dev):
        st = getattr(_lib.lib(), entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                        B, Hq, Hkv, N, d, 1 if causal else 0, float(scale), _stream_handle(dev))
    _lib.check(st, entry)
    return out, lse


_FP8_DTYPES = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))


def _fp8_args(q, k, v, q_scale, k_scale, v_scale, out, lse, causal, scale):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor")
        if t.dtype not in _FP8_DTYPES:
            raise TypeError(f"{name} must hold E4M3 codes (torch.float8_e4m3fn or uint8; got {t.dtype})")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape:
        raise ValueError(f"k and v must be [B,Hkv,N,d] = {(B, Hkv, N, d)}; got {tuple(k.shape)}, {tuple(v.shape)}")
    _check_bf16("out", out, 4)
    if out.shape != q.shape:
        raise ValueError("out must match q's shape")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,Hq,N] tensor")
    _one_device(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return (q.data_ptr(), k.data_ptr(), v.data_ptr(), float(q_scale), float(k_scale), float(v_scale),
            out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d, 1 if causal else 0, float(scale))


def fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_scale: float, k_scale: float, v_scale: float,
            causal: bool = False, scale: float | None = None, out: torch.Tensor | None = None,
            lse: torch.Tensor | None = None):
    """FP8 attention forward (d = 64 or 128): q [B,Hq,N,d], k/v [B,Hkv,N,d] of OCP E4M3 codes
    (torch.float8_e4m3fn or uint8) whose values are q_scale*q, k_scale*k, v_scale*v
    -> (o [B,Hq,N,d] bf16, lse [B,Hq,N] fp32)."""
    B, Hq, N, _ = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    args = _fp8_args(q, k, v, q_scale, k_scale, v_scale, out, lse, causal, scale)
    with torch.cuda.device(q.device):
        st = _lib.lib().fa_fwd_fp8(*args, _stream_handle(q.device))
    _lib.check(st, "fa_fwd_fp8")
    return out, lse


def prepare_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, out, lse, causal: bool = False,
                    scale: float | None = None):
    """Like prepare_fwd, for fwd_fp8 (one fa_fwd_fp8_ws call per invocation)."""
    args = _fp8_args(q, k, v, q_scale, k_scale, v_scale, out, lse, causal, scale)
    B, Hq, N, d = q.shape
    device = q.device
    with torch.cuda.device(device):
        need = fwd_workspace_bytes(B, Hq, N, d)
    ws = torch.empty(need, dtype=torch.uint8, device=device) if need else None
    fn = _lib.lib().fa_fwd_fp8_ws
    tail = (ws.data_ptr() if ws is not None else None, need)

    def call():
        with torch.cuda.device(device):
            st = fn(*args, *tail, torch.cuda.current_stream(device).cuda_stream)
        if st:
            _lib.check(st, "fa_fwd_fp8_ws")
    call.workspace = ws
    return call


def fwd_workspace_bytes(B: int, Hq: int, N: int, d: int) -> int:
    """Workspace fa_fwd_ws needs on the current device (0: single launch)."""
    return int(_lib.lib().fa_fwd_workspace_bytes(B, Hq, N, d))


def decode_workspace_bytes(B: int, Hq: int, L: int, d: int, num_splits: int) -> int:
    return int(_lib.lib().fa_decode_workspace_bytes(B, Hq, L, d, num_splits))


def _check_workspace(ws) -> None:
    """A caller's workspace is handed over as (pointer, bytes): it must be one contiguous block."""
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")


def _check_lens(seq_lens: torch.Tensor, B: int, device) -> None:
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    if seq_lens.device != device:
        raise ValueError("seq_lens must be on the same GPU as q")


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, num_splits: int = 16,
           scale: float | None = None, workspace: torch.Tensor | None = None,
           out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
           seq_lens: torch.Tensor | None = None):
    """Split-KV decode. q [B,Hq,1,d], k/v [B,Hkv,L,d] bf16 -> (o [B,Hq,1,d] bf16, lse [B,Hq] fp32).

    With seq_lens (int32 [B] on the GPU), sequence b attends to its first
    seq_lens[b] keys only (clamped to [0, L]); the rest of its cache rows are
    never read.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t, 4)
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per sequence: q must be [B,Hq,1,d]")
    Hkv, L = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, L, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B,Hkv,L,d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_bytes(B, Hq, L, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_bf16("out", out, 4)
    if out.shape != q.shape:
        raise ValueError("out must match q's shape [B,Hq,1,d]")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,Hq] tensor")
    _check_workspace(workspace)
    _one_device(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse), ("workspace", workspace),
                ("seq_lens", seq_lens))
    with torch.cuda.device(q.device):
        return _decode_call(q, k, v, out, lse, workspace, seq_lens, B, Hq, Hkv, L, d, num_splits, scale)


def _decode_call(q, k, v, out, lse, workspace, seq_lens, B, Hq, Hkv, L, d, num_splits, scale):
    if seq_lens is None:
        st = _lib.lib().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  B, Hq, Hkv, L, d, num_splits, float(scale), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), _stream_handle(q.device))
        _lib.check(st, "fa_decode")
    else:
        _check_lens(seq_lens, B, q.device)
        st = _lib.lib().fa_decode_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                         seq_lens.data_ptr(), B, Hq, Hkv, L, d, num_splits, float(scale),
                                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                         _stream_handle(q.device))
        _lib.check(st, "fa_decode_varlen")
    return out, lse


def bwd_workspace_bytes(B: int, Hq: int, N: int, d: int) -> int:
    return int(_lib.lib().fa_bwd_workspace_bytes(B, Hq, N, d))


def _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, workspace):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_bf16(name, t, 4)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or dk.shape != k.shape or dv.shape != k.shape:
        raise ValueError("k, v, dk, dv must be [B,Hkv,N,d]")
    if o.shape != q.shape or dout.shape != q.shape or dq.shape != q.shape:
        raise ValueError("o, dout, dq must be [B,Hq,N,d]")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,Hq,N] tensor")
    _check_workspace(workspace)
    _one_device(("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout), ("dq", dq), ("dk", dk),
                ("dv", dv), ("workspace", workspace))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, d, int(bool(causal)), float(scale),
            workspace.data_ptr(), workspace.numel() * workspace.element_size())


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, causal: bool = False, scale: float | None = None,
        workspace: torch.Tensor | None = None):
    """Backward pass of fwd (d = 64 or 128): (dq [B,Hq,N,d], dk, dv [B,Hkv,N,d]) bf16, from the
    forward's o and lse and the upstream gradient dout."""
    B, Hq, N, d = q.shape
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(B, Hq, N, d), 16), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    args = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, workspace)
    with torch.cuda.device(q.device):
        st = _lib.lib().fa_bwd(*args, _stream_handle(q.device))
    _lib.check(st, "fa_bwd")
    return dq, dk, dv


def prepare_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal: bool = False, scale: float | None = None):
    """Like prepare_fwd, for the backward pass with caller-owned outputs and workspace."""
    args = _bwd_args(q, k, v, o, lse, dout, dq, dk, dv, causal, scale, workspace)
    fn = _lib.lib().fa_bwd
    device = q.device

    def call():
        with torch.cuda.device(device):
            st = fn(*args, torch.cuda.current_stream(device).cuda_stream)
        if st:
            _lib.check(st, "fa_bwd")
    return call


def prepare_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                causal: bool = False, scale: float | None = None):
    """Check the arguments once and return a callable that re-issues the same
    forward with the least host work: one C call (fa_fwd_ws) on the current
    stream, with a workspace allocated here once when the keys are split.
    call(after_attention=ev) makes that call through fa_fwd_ws_timed, which
    records the torch.cuda.Event `ev` right after the attention kernel (before
    the key-split merge).

    The tensors must stay alive and unmoved while the callable is used.
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_bf16(name, t, 4)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != k.shape or out.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v and out")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,Hq,N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    device = _one_device(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse))
    fn = _lib.lib().fa_fwd_ws
    fn_timed = _lib.lib().fa_fwd_ws_timed
    with torch.cuda.device(device):
        need = fwd_workspace_bytes(B, Hq, N, d)
    ws = torch.empty(need, dtype=torch.uint8, device=device) if need else None
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            B, Hq, Hkv, N, d, 1 if causal else 0, float(scale), ws.data_ptr() if ws is not None else None, need)

    def call(after_attention: torch.cuda.Event | None = None):
        with torch.cuda.device(device):
            stream = torch.cuda.current_stream(device)
            if after_attention is None:
                st = fn(*args, stream.cuda_stream)
                name = "fa_fwd_ws"
            else:
                if not after_attention.cuda_event:  # torch creates the HIP event at its first record
                    after_attention.record(stream)
                st = fn_timed(*args, stream.cuda_stream, after_attention.cuda_event)
                name = "fa_fwd_ws_timed"
        if st:
            _lib.check(st, name)
    call.workspace = ws  # keeps the buffer alive with the callable
    return call


def prepare_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                   workspace: torch.Tensor, num_splits: int = 16, scale: float | None = None,
                   seq_lens: torch.Tensor | None = None):
    """Like prepare_fwd, for split-KV decode with a caller-owned workspace
    (and, with seq_lens, per-sequence key counts as in decode)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_bf16(name, t, 4)
    B, Hq, one, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    if one != 1 or k.shape != (B, Hkv, L, d) or v.shape != k.shape or out.shape != q.shape:
        raise ValueError("decode shapes: q,out [B,Hq,1,d], k,v [B,Hkv,L,d]")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,Hq] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_workspace(workspace)
    _one_device(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse), ("workspace", workspace),
                ("seq_lens", seq_lens))
    if seq_lens is None:
        fn, name = _lib.lib().fa_decode, "fa_decode"
        head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    else:
        _check_lens(seq_lens, B, q.device)
        fn, name = _lib.lib().fa_decode_varlen, "fa_decode_varlen"
        head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), seq_lens.data_ptr())
    args = head + (B, Hq, Hkv, L, d, num_splits, float(scale), workspace.data_ptr(),
                   workspace.numel() * workspace.element_size())
    device = q.device

    def call():
        with torch.cuda.device(device):
            st = fn(*args, torch.cuda.current_stream(device).cuda_stream)
        if st:
            _lib.check(st, name)
    return call


class _Attention(torch.autograd.Function):
    """fwd in the forward pass; bwd (from the saved O and lse) in the backward pass."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = fwd(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal = causal
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              scale: float | None = None) -> torch.Tensor:
    """Differentiable attention: O = softmax(scale Q K^T) V (bf16 [B,Hq,N,d]) through
    torch.autograd; gradients come from the library's backward pass."""
    return _Attention.apply(q, k, v, bool(causal), scale)
