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

THA_OK, THA_ERR_INVALID, THA_ERR_UNSUPPORTED, THA_ERR_HIP, THA_ERR_TOO_LARGE = 0, -1, -2, -3, -4
THA_F32, THA_BF16 = 0, 1
THA_MASK_NONE, THA_MASK_CAUSAL, THA_MASK_KEY_PADDING = 0, 1, 2
THA_ACCUMULATE = 4
THA_KERNEL_AUTO, THA_KERNEL_NARROW, THA_KERNEL_WIDE, THA_KERNEL_SPLIT, THA_KERNEL_SPLIT64 = 0, 1 << 3, 2 << 3, 3 << 3, 4 << 3
THA_MAX_PARTS = THA_MAX_SHARDS = 64
THA_MAX_PERMUTE_TENSORS = 4
THA_NOALLOC_MAX_DELTA = 4 * 1024 * 1024
_KERNELS = {None: THA_KERNEL_AUTO, "auto": THA_KERNEL_AUTO, "narrow": THA_KERNEL_NARROW,
            "wide": THA_KERNEL_WIDE, "split": THA_KERNEL_SPLIT, "split64": THA_KERNEL_SPLIT64}

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
    lib.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_uint, cll,
                                     cll, vp, ctypes.c_float, vp]
    lib.attn_merge_lse.argtypes = [ci, vp, vp, ci, vp, ci, vp, ci, ci, ci, ci, vp]
    lib.shard_permute.argtypes = [vp, ci, ci, vp, ci, ci, ci, ci, ci, vp]
    lib.shard_unpermute.argtypes = [vp, ci, ci, vp, ci, ci, ci, ci, ci, vp]
    lib.shard_all_to_all.argtypes = [vp, ci, ci, vp, ci, vp, ci, ci, ci, vp]
    lib.shard_permute_n.argtypes = [ci, vp, ci, ci, vp, ci, ci, ci, ci, ci, vp]
    lib.shard_unpermute_n.argtypes = [ci, vp, ci, ci, vp, ci, ci, ci, ci, ci, vp]
    for f in (lib.attn_fwd, lib.attn_fwd_ex, lib.attn_bwd, lib.attn_bwd_noalloc, lib.attn_merge_lse, lib.shard_permute,
              lib.shard_unpermute, lib.shard_all_to_all, lib.shard_permute_n, lib.shard_unpermute_n, lib.tha_version):
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
    if rc == THA_ERR_TOO_LARGE:
        raise ValueError(f"{what}: {status_string(rc)}")
    raise ThaError(rc, what)


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return THA_BF16
    if t == torch.float32:
        return THA_F32
    raise NotImplementedError(f"unsupported dtype {t}")


def _is_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not _is_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# The C ABI sees raw pointers only, so every tensor's shape, dtype and device is checked here,
# before any library call: a mismatch would otherwise read or write outside its buffer.
def _expect(t: torch.Tensor, name: str, shape, dtype=None, device=None, dtypes=None):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _bshd(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, S, H, D], got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _kv_len_arg(kv_len, B: int, device):
    if kv_len is None:
        return 0, None
    kv_len = _dev(kv_len, "kv_len")
    _expect(kv_len, "kv_len", (B,), torch.int32, device)
    return THA_MASK_KEY_PADDING, kv_len.data_ptr()


def _kernel_flag(kernel) -> int:
    if kernel not in _KERNELS:
        raise ValueError(f"kernel must be one of {sorted(k for k in _KERNELS if k)} or None, got {kernel!r}")
    return _KERNELS[kernel]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptrs(ts: Sequence[torch.Tensor]):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
             kv_len: Optional[torch.Tensor] = None, q_pos0: int = 0, k_pos0: int = 0,
             scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             return_lse: bool = True, kernel: Optional[str] = None):
    """out [B,Sq,H,D], lse [B,H,Sq] (fp32) = attention of q against k/v (see tha.h attn_fwd).
    kernel: None (automatic) or "narrow" / "wide" / "split" / "split64" to force the form of the bf16
    head-size-128 kernel (attn_fwd_ex's THA_KERNEL_* flags)."""
    load_library()
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    B, Sq, H, D = _bshd(q, "q")
    Sk = _bshd(k, "k")[1]
    _expect(k, "k", (B, Sk, H, D), q.dtype, q.device)
    _expect(v, "v", (B, Sk, H, D), q.dtype, q.device)
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=out_dtype or q.dtype, device=q.device)
    _expect(_dev(out, "out"), "out", (B, Sq, H, D), None, q.device, (torch.bfloat16, torch.float32))
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(_dev(lse, "lse"), "lse", (B, H, Sq), torch.float32, q.device)
    kflag, kvp = _kv_len_arg(kv_len, B, q.device)
    flags = (THA_MASK_CAUSAL if causal else 0) | kflag
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kf = _kernel_flag(kernel)
    lp = lse.data_ptr() if lse is not None else None
    if kf == THA_KERNEL_AUTO:
        rc = _lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dt(out.dtype), lp,
                           B, Sq, Sk, H, D, _dt(q.dtype), flags, int(q_pos0), int(k_pos0), kvp, float(scale),
                           _stream(q))
    else:
        rc = _lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dt(out.dtype), lp,
                              B, Sq, Sk, H, D, _dt(q.dtype), flags | kf, int(q_pos0), int(k_pos0), kvp,
                              float(scale), None, _stream(q))
    _check(rc, "attn_fwd")
    return (out, lse) if return_lse else out


def _view_strides(t: torch.Tensor, name: str):
    """(batch, token) element strides of a [B, S, H, D] view with heads and dims contiguous."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not _is_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 4 or t.stride(3) != 1 or t.stride(2) != t.shape[3]:
        raise ValueError(f"{name} must be a [B, S, H, D] view with contiguous heads and dims")
    return t.stride(0), t.stride(1)


def attn_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                kv_len: Optional[torch.Tensor] = None, q_pos0: int = 0, k_pos0: int = 0,
                scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                accumulate: bool = False, kernel: Optional[str] = None):
    """attn_fwd on strided views (e.g. packed QKV [B,S,3,H,D] split into q, k, v; head subsets),
    and with accumulate=True the fused Ring step: out (fp32) and lse hold a running result over
    other keys and this call merges its own result into them (see tha.h attn_fwd_ex).
    kernel: as attn_fwd.  Returns (out, lse)."""
    load_library()
    strides = list(_view_strides(q, "q"))
    B, Sq, H, D = q.shape
    strides += _view_strides(k, "k")
    Sk = k.shape[1]
    _expect(k, "k", (B, Sk, H, D), q.dtype, q.device)
    strides += _view_strides(v, "v")
    _expect(v, "v", (B, Sk, H, D), q.dtype, q.device)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs the running out and lse")
        out = torch.empty((B, Sq, H, D), dtype=out_dtype or q.dtype, device=q.device)
    if lse is None:
        if accumulate:
            raise ValueError("accumulate needs the running out and lse")
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    strides += _view_strides(out, "out")
    _expect(out, "out", (B, Sq, H, D), None, q.device, (torch.bfloat16, torch.float32))
    _expect(_dev(lse, "lse"), "lse", (B, H, Sq), torch.float32, q.device)
    st = (ctypes.c_longlong * 8)(*strides)
    kflag, kvp = _kv_len_arg(kv_len, B, q.device)
    flags = (THA_MASK_CAUSAL if causal else 0) | (THA_ACCUMULATE if accumulate else 0) | kflag
    flags |= _kernel_flag(kernel)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = _lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _dt(out.dtype), lse.data_ptr(),
                          B, Sq, Sk, H, D, _dt(q.dtype), flags, int(q_pos0), int(k_pos0), kvp, float(scale), st,
                          _stream(q))
    _check(rc, "attn_fwd_ex")
    return out, lse


def _bwd_args(q, k, v, o, dout, lse, kv_len, dq, dk, dv):
    q, k, v, o, dout, lse = (_dev(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"),
                                                        (lse, "lse")))
    B, Sq, H, D = _bshd(q, "q")
    Sk = _bshd(k, "k")[1]
    dev = q.device
    _expect(k, "k", (B, Sk, H, D), q.dtype, dev)
    _expect(v, "v", (B, Sk, H, D), q.dtype, dev)
    _expect(o, "o", (B, Sq, H, D), q.dtype, dev)
    _expect(dout, "dout", (B, Sq, H, D), q.dtype, dev)
    _expect(lse, "lse", (B, H, Sq), torch.float32, dev)
    if dq is None:
        dq = torch.zeros((B, Sq, H, D), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.zeros((B, Sk, H, D), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.zeros((B, Sk, H, D), dtype=torch.float32, device=dev)
    for t, n, S_ in ((dq, "dq", Sq), (dk, "dk", Sk), (dv, "dv", Sk)):
        _expect(_dev(t, n), n, (B, S_, H, D), torch.float32, dev)
    kflag, kvp = _kv_len_arg(kv_len, B, dev)
    return (B, Sq, Sk, H, D), (q, k, v, o, dout, lse), (dq, dk, dv), kflag, kvp


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
             lse: torch.Tensor, *, causal: bool = False, kv_len: Optional[torch.Tensor] = None, q_pos0: int = 0,
             k_pos0: int = 0, scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None):
    """Gradients of attn_fwd (see tha.h attn_bwd): returns (dq, dk, dv), fp32.  Given dq / dk / dv
    are accumulated into; missing ones start from zero.  workspace: fp32 of >= B*H*Sq elements."""
    load_library()
    (B, Sq, Sk, H, D), (q, k, v, o, dout, lse), (dq, dk, dv), kflag, kvp = _bwd_args(q, k, v, o, dout, lse, kv_len,
                                                                                      dq, dk, dv)
    if workspace is None:
        workspace = torch.empty((B * H * Sq,), dtype=torch.float32, device=q.device)
    _dev(workspace, "workspace")
    if workspace.dtype != torch.float32 or workspace.numel() < B * H * Sq or workspace.device != q.device:
        raise ValueError("workspace must be float32 on q's device with at least B*H*Sq elements")
    flags = (THA_MASK_CAUSAL if causal else 0) | kflag
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = _lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, Sq, Sk, H, D,
                       _dt(q.dtype), flags, int(q_pos0), int(k_pos0), kvp, float(scale), _stream(q))
    _check(rc, "attn_bwd")
    return dq, dk, dv


def attn_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
                     lse: torch.Tensor, *, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                     causal: bool = False, kv_len: Optional[torch.Tensor] = None, q_pos0: int = 0, k_pos0: int = 0,
                     scale: Optional[float] = None):
    """attn_bwd without a workspace (see tha.h attn_bwd_noalloc): the library's fixed per-device
    scratch holds Delta, so the call allocates nothing; the caller passes the fp32 dq, dk, dv to
    accumulate into.  B*H*Sq must not exceed THA_NOALLOC_MAX_DELTA.  Overlapping calls on one device
    race on that scratch."""
    load_library()
    (B, Sq, Sk, H, D), (q, k, v, o, dout, lse), (dq, dk, dv), kflag, kvp = _bwd_args(q, k, v, o, dout, lse, kv_len,
                                                                                      dq, dk, dv)
    flags = (THA_MASK_CAUSAL if causal else 0) | kflag
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = _lib.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                               lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Sq, Sk, H, D,
                               _dt(q.dtype), flags, int(q_pos0), int(k_pos0), kvp, float(scale), _stream(q))
    _check(rc, "attn_bwd_noalloc")
    return dq, dk, dv


def attn_merge_lse(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor], *,
                   out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                   lse_out: Optional[torch.Tensor] = None, return_lse: bool = True):
    """Log-sum-exp merge of partial results (see tha.h attn_merge_lse)."""
    load_library()
    if len(o_parts) != len(lse_parts) or len(o_parts) == 0:
        raise ValueError("need matching, non-empty o_parts and lse_parts")
    if len(o_parts) > THA_MAX_PARTS:
        raise ValueError(f"at most {THA_MAX_PARTS} parts")
    o0 = _dev(o_parts[0], "o_parts[0]")
    B, S, H, D = _bshd(o0, "o_parts[0]")
    dev = o0.device
    for i, (o, l) in enumerate(zip(o_parts, lse_parts)):
        _expect(_dev(o, f"o_parts[{i}]"), f"o_parts[{i}]", (B, S, H, D), o0.dtype, dev)
        _expect(_dev(l, f"lse_parts[{i}]"), f"lse_parts[{i}]", (B, H, S), torch.float32, dev)
    part_dt = _dt(o0.dtype)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=out_dtype or o0.dtype, device=dev)
    _expect(_dev(out, "out"), "out", (B, S, H, D), None, dev, (torch.bfloat16, torch.float32))
    if lse_out is None and return_lse:
        lse_out = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    if lse_out is not None:
        _expect(_dev(lse_out, "lse_out"), "lse_out", (B, H, S), torch.float32, dev)
    rc = _lib.attn_merge_lse(len(o_parts), _ptrs(o_parts), _ptrs(lse_parts), part_dt, out.data_ptr(),
                             _dt(out.dtype), lse_out.data_ptr() if lse_out is not None else None, B, S, H, D,
                             _stream(out))
    _check(rc, "attn_merge_lse")
    return (out, lse_out) if return_lse else out


def _shard_list(shards: Sequence[torch.Tensor], name: str):
    shards = [_dev(s, f"{name}[{i}]") for i, s in enumerate(shards)]
    if not shards or len(shards) > THA_MAX_SHARDS:
        raise ValueError(f"need 1 to {THA_MAX_SHARDS} {name}")
    for i, s in enumerate(shards[1:], 1):
        _expect(s, f"{name}[{i}]", shards[0].shape, shards[0].dtype, shards[0].device)
    return shards


def shard_permute(shards: Sequence[torch.Tensor], group: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """P sequence shards [B,S/P,H,D] -> head group `group` over the whole sequence [B,S,H/P,D]."""
    load_library()
    shards = _shard_list(shards, "shards")
    P = len(shards)
    B, Sl, H, D = _bshd(shards[0], "shards[0]")
    if H % P:
        raise ValueError(f"heads ({H}) must be divisible by the shard count ({P})")
    if out is None:
        out = torch.empty((B, Sl * P, H // P, D), dtype=shards[0].dtype, device=shards[0].device)
    _expect(_dev(out, "out"), "out", (B, Sl * P, H // P, D), shards[0].dtype, shards[0].device)
    rc = _lib.shard_permute(_ptrs(shards), P, int(group), out.data_ptr(), B, Sl * P, H, D,
                            shards[0].element_size(), _stream(out))
    _check(rc, "shard_permute")
    return out


def shard_unpermute(x: torch.Tensor, group: int, shards: Sequence[torch.Tensor]) -> None:
    """Write head group `group` of x [B,S,H/P,D] back into the P sequence shards [B,S/P,H,D]."""
    load_library()
    x = _dev(x, "x")
    shards = _shard_list(shards, "shards")
    P = len(shards)
    B, S, Hl, D = _bshd(x, "x")
    if S % P:
        raise ValueError(f"sequence length ({S}) must be divisible by the shard count ({P})")
    _expect(shards[0], "shards[0]", (B, S // P, Hl * P, D), x.dtype, x.device)
    rc = _lib.shard_unpermute(x.data_ptr(), P, int(group), _ptrs(shards), B, S, Hl * P, D, x.element_size(),
                              _stream(x))
    _check(rc, "shard_unpermute")


def shard_permute_n(shard_sets: Sequence[Sequence[torch.Tensor]], group: int,
                    outs: Optional[Sequence[torch.Tensor]] = None) -> list:
    """shard_permute of n tensors of one shape (e.g. the Q, K and V shards of a Ulysses step) in one
    launch: shard_sets[t] are the P sequence shards [B,S/P,H,D] of tensor t.  Returns the n grouped
    tensors [B,S,H/P,D] (bit-identical to n shard_permute calls)."""
    load_library()
    n = len(shard_sets)
    if not 1 <= n <= THA_MAX_PERMUTE_TENSORS:
        raise ValueError(f"need 1 to {THA_MAX_PERMUTE_TENSORS} tensors")
    sets = [_shard_list(ss, f"shard_sets[{t}]") for t, ss in enumerate(shard_sets)]
    P = len(sets[0])
    first = sets[0][0]
    for t, ss in enumerate(sets):
        if len(ss) != P:
            raise ValueError("every tensor needs the same number of shards")
        _expect(ss[0], f"shard_sets[{t}][0]", first.shape, first.dtype, first.device)
    B, Sl, H, D = _bshd(first, "shard_sets[0][0]")
    if H % P:
        raise ValueError(f"heads ({H}) must be divisible by the shard count ({P})")
    shape = (B, Sl * P, H // P, D)
    if outs is None:
        outs = [torch.empty(shape, dtype=first.dtype, device=first.device) for _ in range(n)]
    if len(outs) != n:
        raise ValueError("need one output per tensor")
    for t, o in enumerate(outs):
        _expect(_dev(o, f"outs[{t}]"), f"outs[{t}]", shape, first.dtype, first.device)
    rc = _lib.shard_permute_n(n, _ptrs([x for ss in sets for x in ss]), P, int(group), _ptrs(outs), B, Sl * P, H, D,
                              first.element_size(), _stream(first))
    _check(rc, "shard_permute_n")
    return list(outs)


def shard_unpermute_n(xs: Sequence[torch.Tensor], group: int, shard_sets: Sequence[Sequence[torch.Tensor]]) -> None:
    """shard_unpermute of n tensors in one launch: head group `group` of xs[t] [B,S,H/P,D] is written
    back into the P sequence shards shard_sets[t] [B,S/P,H,D]."""
    load_library()
    n = len(xs)
    if not 1 <= n <= THA_MAX_PERMUTE_TENSORS or len(shard_sets) != n:
        raise ValueError(f"need 1 to {THA_MAX_PERMUTE_TENSORS} tensors, with one shard set each")
    xs = [_dev(x, f"xs[{t}]") for t, x in enumerate(xs)]
    B, S, Hl, D = _bshd(xs[0], "xs[0]")
    sets = [_shard_list(ss, f"shard_sets[{t}]") for t, ss in enumerate(shard_sets)]
    P = len(sets[0])
    if S % P:
        raise ValueError(f"sequence length ({S}) must be divisible by the shard count ({P})")
    for t in range(n):
        _expect(xs[t], f"xs[{t}]", (B, S, Hl, D), xs[0].dtype, xs[0].device)
        if len(sets[t]) != P:
            raise ValueError("every tensor needs the same number of shards")
        _expect(sets[t][0], f"shard_sets[{t}][0]", (B, S // P, Hl * P, D), xs[0].dtype, xs[0].device)
    rc = _lib.shard_unpermute_n(n, _ptrs(xs), P, int(group), _ptrs([x for ss in sets for x in ss]), B, S, Hl * P, D,
                                xs[0].element_size(), _stream(xs[0]))
    _check(rc, "shard_unpermute_n")


def shard_all_to_all(inputs: Sequence[torch.Tensor], rank: int, scatter_dim: int, gather_dim: int,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """What rank `rank` holds after an all-to-all of the P ranks' tensors `inputs` (one shape and
    dtype, contiguous): each split into P chunks along scatter_dim, chunk r sent to rank r, the
    received chunks concatenated in rank order along gather_dim (see tha.h shard_all_to_all).
    Negative dims count from the end."""
    load_library()
    inputs = _shard_list(inputs, "inputs")
    P = len(inputs)
    shape = list(inputs[0].shape)
    nd = len(shape)
    if not 1 <= nd <= 8:
        raise ValueError("inputs must have 1 to 8 dims")
    sd, gd = int(scatter_dim), int(gather_dim)
    if not (-nd <= sd < nd and -nd <= gd < nd):
        raise ValueError(f"scatter_dim / gather_dim out of range for {nd} dims")
    sd, gd = sd % nd, gd % nd
    if sd == gd:
        raise ValueError("scatter_dim and gather_dim must differ")
    if shape[sd] % P:
        raise ValueError(f"size {shape[sd]} of the scatter dim is not divisible by the rank count {P}")
    out_shape = list(shape)
    out_shape[sd] //= P
    out_shape[gd] *= P
    if out is None:
        out = torch.empty(out_shape, dtype=inputs[0].dtype, device=inputs[0].device)
    _expect(_dev(out, "out"), "out", out_shape, inputs[0].dtype, inputs[0].device)
    sh = (ctypes.c_longlong * nd)(*shape)
    rc = _lib.shard_all_to_all(_ptrs(inputs), P, int(rank), out.data_ptr(), nd, sh, sd, gd,
                               inputs[0].element_size(), _stream(out))
    _check(rc, "shard_all_to_all")
    return out


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
                  kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                  kernel: Optional[str] = None):
    """One GPU's Ulysses share: the P sequence shards [B,S/P,H,D] of Q, K and V are permuted to head
    group `group` over the whole sequence (one shard_permute_n launch) and attended (attn_fwd).
    Returns (out [B,S,H/P,D], lse [B,H/P,S])."""
    q, k, v = shard_permute_n([q_shards, k_shards, v_shards], group)
    return attn_fwd(q, k, v, causal=causal, kv_len=kv_len, scale=scale, kernel=kernel)


def ring_share(q: torch.Tensor, k_chunks: Sequence[torch.Tensor], v_chunks: Sequence[torch.Tensor], *,
               q_pos0: int, k_pos0s: Sequence[int], causal: bool = True, scale: Optional[float] = None,
               fused: bool = True, out_dtype: Optional[torch.dtype] = None, kernel: Optional[str] = None):
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
                        accumulate=True, kernel=kernel)
        return attn_merge_lse([o], [lse], out_dtype=out_dtype or q.dtype)
    parts = [attn_fwd(q, kc, vc, causal=causal, q_pos0=q_pos0, k_pos0=kp, scale=scale, out_dtype=torch.float32,
                      kernel=kernel) for kc, vc, kp in zip(k_chunks, v_chunks, k_pos0s)]
    return attn_merge_lse([p[0] for p in parts], [p[1] for p in parts], out_dtype=out_dtype or q.dtype)
