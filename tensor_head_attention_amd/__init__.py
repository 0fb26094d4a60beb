"""Python binding of libtha.so (the C ABI declared in include/tha.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if libtha.so is missing or fails to load, every call
raises.  Build it with `python -m tensor_head_attention_amd.build`.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtha.so")

THA_OK, THA_ERR_INVALID, THA_ERR_UNSUPPORTED, THA_ERR_HIP = 0, -1, -2, -3
THA_F32, THA_BF16 = 0, 1
THA_MASK_NONE, THA_MASK_CAUSAL, THA_MASK_KEY_PADDING = 0, 1, 2
THA_ACCUMULATE = 4
THA_MAX_PARTS = THA_MAX_SHARDS = 64

_lib = None


class ThaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status) if _lib is not None else status} (status {status})")


def load_library(path: str = LIB_PATH):
    """Load libtha.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m tensor_head_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, ci, cll = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, ci, vp, ci, ci, ci, ci, ci, ci, ctypes.c_uint, cll, cll, vp,
                             ctypes.c_float, vp]
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, ci, vp, ci, ci, ci, ci, ci, ci, ctypes.c_uint, cll, cll, vp,
                                ctypes.c_float, vp, vp]
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_uint, cll, cll,
                             vp, ctypes.c_float, vp]
    lib.attn_merge_lse.argtypes = [ci, vp, vp, ci, vp, ci, vp, ci, ci, ci, ci, vp]
    lib.shard_permute.argtypes = [vp, ci, ci, vp, ci, ci, ci, ci, ci, vp]
    lib.shard_unpermute.argtypes = [vp, ci, ci, vp, ci, ci, ci, ci, ci, vp]
    for f in (lib.attn_fwd, lib.attn_fwd_ex, lib.attn_bwd, lib.attn_merge_lse, lib.shard_permute, lib.shard_unpermute,
              lib.tha_version):
        f.restype = ci
    lib.tha_status_string.argtypes = [ci]
    lib.tha_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().tha_status_string(int(status)).decode()


def version() -> int:
    return load_library().tha_version()


def _check(rc: int, what: str):
    if rc == THA_OK:
        return
    if rc == THA_ERR_INVALID:
        raise ValueError(f"{what}: {status_string(rc)}")
    if rc == THA_ERR_UNSUPPORTED:
        raise NotImplementedError(f"{what}: {status_string(rc)}")
    raise ThaError(rc, what)


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return THA_BF16
    if t == torch.float32:
        return THA_F32
    raise NotImplementedError(f"unsupported dtype {t}")


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptrs(ts: Sequence[torch.Tensor]):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
             kv_len: Optional[torch.Tensor] = None, q_pos0: int = 0, k_pos0: int = 0,
             scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             return_lse: bool = True):
    """out [B,Sq,H,D], lse [B,H,Sq] (fp32) = attention of q against k/v (see tha.h attn_fwd)."""
    load_library()
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=out_dtype or q.dtype, device=q.device)
    _dev(out, "out")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    flags = THA_MASK_CAUSAL if causal else 0
    kvp = None
    if kv_len is not None:
        kv_len = _dev(kv_len, "kv_len")
        if kv_len.dtype != torch.int32:
            raise ValueError("kv_len must be int32")
        flags |= THA_MASK_KEY_PADDING
        kvp = kv_len.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = _lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dt(out.dtype),
                       lse.data_ptr() if lse is not None else None, B, Sq, Sk, H, D, _dt(q.dtype), flags,
                       int(q_pos0), int(k_pos0), kvp, float(scale), _stream(q))
    _check(rc, "attn_fwd")
    return (out, lse) if return_lse else out


def _view_strides(t: torch.Tensor, name: str):
    """(batch, token) element strides of a [B, S, H, D] view with heads and dims contiguous."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 4 or t.stride(3) != 1 or t.stride(2) != t.shape[3]:
        raise ValueError(f"{name} must be a [B, S, H, D] view with contiguous heads and dims")
    return t.stride(0), t.stride(1)


def attn_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                kv_len: Optional[torch.Tensor] = None, q_pos0: int = 0, k_pos0: int = 0,
                scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                accumulate: bool = False):
    """attn_fwd on strided views (e.g. packed QKV [B,S,3,H,D] split into q, k, v; head subsets),
    and with accumulate=True the fused Ring step: out (fp32) and lse hold a running result over
    other keys and this call merges its own result into them (see tha.h attn_fwd_ex).
    Returns (out, lse)."""
    load_library()
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs the running out and lse")
        out = torch.empty((B, Sq, H, D), dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        if accumulate:
            raise ValueError("accumulate needs the running out and lse")
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _dev(lse, "lse")
    strides = []
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        strides += list(_view_strides(t, n))
    st = (ctypes.c_longlong * 8)(*strides)
    flags = (THA_MASK_CAUSAL if causal else 0) | (THA_ACCUMULATE if accumulate else 0)
    kvp = None
    if kv_len is not None:
        kv_len = _dev(kv_len, "kv_len")
        if kv_len.dtype != torch.int32:
            raise ValueError("kv_len must be int32")
        flags |= THA_MASK_KEY_PADDING
        kvp = kv_len.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = _lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dt(out.dtype), lse.data_ptr(),
                          B, Sq, Sk, H, D, _dt(q.dtype), flags, int(q_pos0), int(k_pos0), kvp, float(scale), st,
                          _stream(q))
    _check(rc, "attn_fwd_ex")
    return out, lse


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
             lse: torch.Tensor, *, causal: bool = False, kv_len: Optional[torch.Tensor] = None, q_pos0: int = 0,
             k_pos0: int = 0, scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None):
    """Gradients of attn_fwd (see tha.h attn_bwd): returns (dq, dk, dv), fp32.  Given dq / dk / dv
    are accumulated into; missing ones start from zero.  workspace: fp32 of >= B*H*Sq elements."""
    load_library()
    q, k, v, o, dout, lse = (_dev(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"),
                                                        (lse, "lse")))
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if lse.dtype != torch.float32:
        raise ValueError("lse must be float32")
    if dq is None:
        dq = torch.zeros((B, Sq, H, D), dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.zeros((B, Sk, H, D), dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.zeros((B, Sk, H, D), dtype=torch.float32, device=q.device)
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _dev(t, n)
        if t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32")
    if workspace is None:
        workspace = torch.empty((B * H * Sq,), dtype=torch.float32, device=q.device)
    if workspace.dtype != torch.float32 or workspace.numel() < B * H * Sq:
        raise ValueError("workspace must be float32 with at least B*H*Sq elements")
    _dev(workspace, "workspace")
    flags = THA_MASK_CAUSAL if causal else 0
    kvp = None
    if kv_len is not None:
        kv_len = _dev(kv_len, "kv_len")
        if kv_len.dtype != torch.int32:
            raise ValueError("kv_len must be int32")
        flags |= THA_MASK_KEY_PADDING
        kvp = kv_len.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = _lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, Sq, Sk, H, D,
                       _dt(q.dtype), flags, int(q_pos0), int(k_pos0), kvp, float(scale), _stream(q))
    _check(rc, "attn_bwd")
    return dq, dk, dv


def attn_merge_lse(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor], *,
                   out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                   lse_out: Optional[torch.Tensor] = None, return_lse: bool = True):
    """Log-sum-exp merge of partial results (see tha.h attn_merge_lse)."""
    load_library()
    if len(o_parts) != len(lse_parts) or len(o_parts) == 0:
        raise ValueError("need matching, non-empty o_parts and lse_parts")
    for i, (o, l) in enumerate(zip(o_parts, lse_parts)):
        _dev(o, f"o_parts[{i}]"), _dev(l, f"lse_parts[{i}]")
        if l.dtype != torch.float32:
            raise ValueError("lse parts must be float32")
    B, S, H, D = o_parts[0].shape
    part_dt = _dt(o_parts[0].dtype)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=out_dtype or o_parts[0].dtype, device=o_parts[0].device)
    if lse_out is None and return_lse:
        lse_out = torch.empty((B, H, S), dtype=torch.float32, device=o_parts[0].device)
    rc = _lib.attn_merge_lse(len(o_parts), _ptrs(o_parts), _ptrs(lse_parts), part_dt, out.data_ptr(),
                             _dt(out.dtype), lse_out.data_ptr() if lse_out is not None else None, B, S, H, D,
                             _stream(out))
    _check(rc, "attn_merge_lse")
    return (out, lse_out) if return_lse else out


def shard_permute(shards: Sequence[torch.Tensor], group: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """P sequence shards [B,S/P,H,D] -> head group `group` over the whole sequence [B,S,H/P,D]."""
    load_library()
    shards = [_dev(s, f"shards[{i}]") for i, s in enumerate(shards)]
    P = len(shards)
    B, Sl, H, D = shards[0].shape
    if out is None:
        out = torch.empty((B, Sl * P, H // P if P else H, D), dtype=shards[0].dtype, device=shards[0].device)
    rc = _lib.shard_permute(_ptrs(shards), P, int(group), _dev(out, "out").data_ptr(), B, Sl * P, H, D,
                            shards[0].element_size(), _stream(out))
    _check(rc, "shard_permute")
    return out


def shard_unpermute(x: torch.Tensor, group: int, shards: Sequence[torch.Tensor]) -> None:
    """Write head group `group` of x [B,S,H/P,D] back into the P sequence shards [B,S/P,H,D]."""
    load_library()
    x = _dev(x, "x")
    shards = [_dev(s, f"shards[{i}]") for i, s in enumerate(shards)]
    P = len(shards)
    B, S, Hl, D = x.shape
    rc = _lib.shard_unpermute(x.data_ptr(), P, int(group), _ptrs(shards), B, S, Hl * P, D, x.element_size(),
                              _stream(x))
    _check(rc, "shard_unpermute")


class _Attention(torch.autograd.Function):
    """Differentiable attention: attn_fwd forward, attn_bwd backward (saved o and lse)."""

    @staticmethod
    def forward(ctx, q, k, v, causal, kv_len, q_pos0, k_pos0, scale):
        o, lse = attn_fwd(q, k, v, causal=causal, kv_len=kv_len, q_pos0=q_pos0, k_pos0=k_pos0, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.kv_len = kv_len
        ctx.opts = (causal, q_pos0, k_pos0, scale)
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse = ctx.saved_tensors
        causal, q_pos0, k_pos0, scale = ctx.opts
        dq, dk, dv = attn_bwd(q, k, v, o, dout.to(q.dtype).contiguous(), lse, causal=causal, kv_len=ctx.kv_len,
                              q_pos0=q_pos0, k_pos0=k_pos0, scale=scale)
        # the gradients are fp32 accumulators; autograd receives them in the inputs' dtype
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
              kv_len: Optional[torch.Tensor] = None, q_pos0: int = 0, k_pos0: int = 0,
              scale: Optional[float] = None) -> torch.Tensor:
    """Attention output [B,Sq,H,D] (dtype of q) with autograd support: the forward runs attn_fwd,
    the backward attn_bwd, both in the library's kernels."""
    return _Attention.apply(q, k, v, causal, kv_len, q_pos0, k_pos0, scale)


def ulysses_share(q_shards: Sequence[torch.Tensor], k_shards: Sequence[torch.Tensor],
                  v_shards: Sequence[torch.Tensor], group: int, *, causal: bool = True,
                  kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None):
    """One GPU's Ulysses share: the P sequence shards [B,S/P,H,D] of Q, K and V are permuted to head
    group `group` over the whole sequence (shard_permute) and attended (attn_fwd).
    Returns (out [B,S,H/P,D], lse [B,H/P,S])."""
    q, k, v = (shard_permute(s, group) for s in (q_shards, k_shards, v_shards))
    return attn_fwd(q, k, v, causal=causal, kv_len=kv_len, scale=scale)


def ring_share(q: torch.Tensor, k_chunks: Sequence[torch.Tensor], v_chunks: Sequence[torch.Tensor], *,
               q_pos0: int, k_pos0s: Sequence[int], causal: bool = True, scale: Optional[float] = None,
               fused: bool = True, out_dtype: Optional[torch.dtype] = None):
    """One GPU's Ring share: the local Q chunk (first query at global position q_pos0) against K/V
    chunks that arrive in turn (first key of chunk t at k_pos0s[t]).  fused=True merges each chunk's
    result into a running fp32 (o, lse) in the attention epilogue (attn_fwd_ex with accumulate);
    fused=False keeps fp32 partials and merges them once (attn_merge_lse).
    Returns (out [B,Sq,H,D] in out_dtype (default q's), lse [B,H,Sq])."""
    if len(k_chunks) != len(v_chunks) or len(k_chunks) != len(k_pos0s) or not k_chunks:
        raise ValueError("need matching, non-empty k_chunks, v_chunks and k_pos0s")
    B, Sq, H, D = q.shape
    if fused:
        o = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
        lse = torch.full((B, H, Sq), float("-inf"), dtype=torch.float32, device=q.device)
        for kc, vc, kp in zip(k_chunks, v_chunks, k_pos0s):
            attn_fwd_ex(q, kc, vc, causal=causal, q_pos0=q_pos0, k_pos0=kp, scale=scale, out=o, lse=lse,
                        accumulate=True)
        return attn_merge_lse([o], [lse], out_dtype=out_dtype or q.dtype)
    parts = [attn_fwd(q, kc, vc, causal=causal, q_pos0=q_pos0, k_pos0=kp, scale=scale, out_dtype=torch.float32)
             for kc, vc, kp in zip(k_chunks, v_chunks, k_pos0s)]
    return attn_merge_lse([p[0] for p in parts], [p[1] for p in parts], out_dtype=out_dtype or q.dtype)
