"""fp64 CPU oracle for one GPU's share of head/sequence-parallel attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library (``tensor_head_attention_amd``) and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, written from
the pages' definitions; see the header of that file for the passages it
follows).  This module only compiles it with gcc and marshals torch CPU
tensors into it.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (always, when force)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_attention.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, ctypes.c_int,
                                         i64, i64, vp, ctypes.c_double, i64, vp, dp, dp, ctypes.c_int]
        lib.oracle_attention_bruteforce.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64,
                                                    ctypes.c_int, i64, i64, vp, ctypes.c_double, dp, dp, dp]
        lib.oracle_merge_lse.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, i64, dp, dp]
        lib.oracle_shard_permute.argtypes = [vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, ctypes.c_int, vp]
        lib.oracle_shard_unpermute.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, ctypes.c_int, vp]
        lib.oracle_attention_backward.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64,
                                                  ctypes.c_int, i64, i64, vp, ctypes.c_double, dp, dp, dp,
                                                  ctypes.c_int]
        lib.oracle_all_to_all.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, vp]
        for f in (lib.oracle_attention, lib.oracle_attention_bruteforce, lib.oracle_merge_lse,
                  lib.oracle_shard_permute, lib.oracle_shard_unpermute, lib.oracle_attention_backward,
                  lib.oracle_all_to_all):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"oracle inputs must be float32 or bfloat16, got {t.dtype}")


def _host(t: torch.Tensor) -> torch.Tensor:
    if t.device.type != "cpu":
        raise ValueError("oracle takes host (CPU) tensors only")
    return t.contiguous()


def _ptr_array(ptrs: Sequence[int]):
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return arr


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
              q_pos0: int = 0, k_pos0: int = 0, kv_len: Optional[torch.Tensor] = None,
              scale: Optional[float] = None, rows: Optional[torch.Tensor] = None,
              nthreads: int = 0):
    """Two-pass fp64 attention.

    q: [B, Sq, H, D]; k, v: [B, Sk, H, D] (float32 or bfloat16, CPU).
    rows: optional int64 tensor of flat row indices b*Sq + i.
    Returns (out, lse) as float64 tensors:
      rows is None -> out [B, Sq, H, D], lse [B, H, Sq]
      rows given   -> out [n, H, D],     lse [n, H]
    """
    q, k, v = _host(q), _host(k), _host(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    B, Sq, H, D = q.shape
    Bk, Sk, Hk, Dk = k.shape
    if (Bk, Hk, Dk) != (B, H, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kl = None
    if kv_len is not None:
        kl = _host(kv_len.to(torch.int32))
    if rows is None:
        n = B * Sq
        out = torch.empty((B * Sq, H, D), dtype=torch.float64)
        lse = torch.empty((B * Sq, H), dtype=torch.float64)
        rp = None
    else:
        rows = _host(rows.to(torch.int64))
        n = rows.numel()
        out = torch.empty((n, H, D), dtype=torch.float64)
        lse = torch.empty((n, H), dtype=torch.float64)
        rp = rows.data_ptr()
    rc = _load().oracle_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), dt, B, Sq, Sk, H, D,
                                  int(bool(causal)), int(q_pos0), int(k_pos0),
                                  kl.data_ptr() if kl is not None else None, float(scale), n, rp,
                                  out.data_ptr(), lse.data_ptr(), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    if rows is None:
        return out.view(B, Sq, H, D), lse.view(B, Sq, H).permute(0, 2, 1).contiguous()
    return out, lse


def attention_backward(q, k, v, dout, *, causal: bool = False, q_pos0: int = 0, k_pos0: int = 0,
                       kv_len: Optional[torch.Tensor] = None, scale: Optional[float] = None, nthreads: int = 0):
    """fp64 gradients (dq, dk, dv) of attention for the cotangent dout (same masks and positions
    as attention()).  q, dout: [B, Sq, H, D]; k, v: [B, Sk, H, D]; float32 or bfloat16, one dtype.
    Returns float64 tensors dq [B, Sq, H, D], dk [B, Sk, H, D], dv [B, Sk, H, D]."""
    q, k, v, dout = _host(q), _host(k), _host(v), _host(dout)
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k, v, dout)):
        raise TypeError("q, k, v, dout must share one dtype")
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if tuple(k.shape) != (B, Sk, H, D) or tuple(v.shape) != tuple(k.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kl = _host(kv_len.to(torch.int32)) if kv_len is not None else None
    dq = torch.empty((B, Sq, H, D), dtype=torch.float64)
    dk = torch.empty((B, Sk, H, D), dtype=torch.float64)
    dv = torch.empty((B, Sk, H, D), dtype=torch.float64)
    rc = _load().oracle_attention_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dt,
                                           B, Sq, Sk, H, D, int(bool(causal)), int(q_pos0), int(k_pos0),
                                           kl.data_ptr() if kl is not None else None, float(scale),
                                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention_backward rejected its arguments")
    return dq, dk, dv


def attention_bruteforce(q, k, v, *, causal=False, q_pos0=0, k_pos0=0, kv_len=None, scale=None):
    """Full-matrix route (no max shift) for tiny shapes: returns (out, lse, P)."""
    q, k, v = _host(q), _host(k), _host(v)
    dt = _dtype_code(q)
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kl = _host(kv_len.to(torch.int32)) if kv_len is not None else None
    out = torch.empty((B, Sq, H, D), dtype=torch.float64)
    lse = torch.empty((B, H, Sq), dtype=torch.float64)
    P = torch.empty((B, H, Sq, Sk), dtype=torch.float64)
    rc = _load().oracle_attention_bruteforce(q.data_ptr(), k.data_ptr(), v.data_ptr(), dt, B, Sq, Sk, H, D,
                                             int(bool(causal)), int(q_pos0), int(k_pos0),
                                             kl.data_ptr() if kl is not None else None, float(scale),
                                             out.data_ptr(), lse.data_ptr(), P.data_ptr())
    if rc != 0:
        raise ValueError("oracle_attention_bruteforce rejected its arguments")
    return out, lse, P


def merge_lse(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor]):
    """Log-sum-exp merge of n partials: o [B, S, H, D], lse [B, H, S] (fp64 math)."""
    if len(o_parts) < 1 or len(o_parts) != len(lse_parts):
        raise ValueError("need n >= 1 matching partials")
    os_ = [_host(o.to(torch.float64)) for o in o_parts]
    ls_ = [_host(l.to(torch.float64)) for l in lse_parts]
    B, S, H, D = os_[0].shape
    out = torch.empty((B, S, H, D), dtype=torch.float64)
    lse = torch.empty((B, H, S), dtype=torch.float64)
    rc = _load().oracle_merge_lse(len(os_), _ptr_array([o.data_ptr() for o in os_]),
                                  _ptr_array([l.data_ptr() for l in ls_]), B, S, H, D,
                                  out.data_ptr(), lse.data_ptr())
    if rc != 0:
        raise ValueError("oracle_merge_lse rejected its arguments")
    return out, lse


def shard_permute(shards: Sequence[torch.Tensor], group: int) -> torch.Tensor:
    """P shards [B, S/P, H, D] -> head group `group` over the full sequence [B, S, H/P, D]."""
    sh = [_host(s) for s in shards]
    P = len(sh)
    B, Sl, H, D = sh[0].shape
    S = Sl * P
    if H % P:
        raise ValueError("H must be divisible by P")
    out = torch.empty((B, S, H // P, D), dtype=sh[0].dtype)
    rc = _load().oracle_shard_permute(_ptr_array([s.data_ptr() for s in sh]), P, int(group), B, S, H, D,
                                      sh[0].element_size(), out.data_ptr())
    if rc != 0:
        raise ValueError("oracle_shard_permute rejected its arguments")
    return out


def shard_unpermute(groups: Sequence[torch.Tensor]):
    """Head-group outputs [B, S, H/P, D] (all P groups) -> P sequence shards [B, S/P, H, D]."""
    gs = [_host(g) for g in groups]
    P = len(gs)
    B, S, Hl, D = gs[0].shape
    H = Hl * P
    shards = [torch.empty((B, S // P, H, D), dtype=gs[0].dtype) for _ in range(P)]
    rc = _load().oracle_shard_unpermute(_ptr_array([g.data_ptr() for g in gs]), P, B, S, H, D,
                                        gs[0].element_size(), _ptr_array([s.data_ptr() for s in shards]))
    if rc != 0:
        raise ValueError("oracle_shard_unpermute rejected its arguments")
    return shards


def all_to_all(inputs: Sequence[torch.Tensor], rank: int, scatter_dim: int, gather_dim: int) -> torch.Tensor:
    """What rank `rank` holds after the all-to-all of the P ranks' tensors `inputs` (one shape, one
    dtype): each input split into P chunks along scatter_dim, chunk r sent to rank r, the received
    chunks concatenated in rank order along gather_dim."""
    ins = [_host(t) for t in inputs]
    P = len(ins)
    shape = list(ins[0].shape)
    if any(list(t.shape) != shape or t.dtype != ins[0].dtype for t in ins):
        raise ValueError("inputs must share one shape and dtype")
    nd = len(shape)
    sd, gd = scatter_dim % nd, gather_dim % nd
    if shape[sd] % P:
        raise ValueError("the scatter dim must be divisible by the rank count")
    out_shape = list(shape)
    out_shape[sd] //= P
    out_shape[gd] *= P
    out = torch.empty(out_shape, dtype=ins[0].dtype)
    sh = (ctypes.c_int64 * nd)(*shape)
    rc = _load().oracle_all_to_all(_ptr_array([t.data_ptr() for t in ins]), P, int(rank), nd, sh, sd, gd,
                                   ins[0].element_size(), out.data_ptr())
    if rc != 0:
        raise ValueError("oracle_all_to_all rejected its arguments")
    return out
