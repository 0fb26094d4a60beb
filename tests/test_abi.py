"""CPU checks of the C-ABI library: it loads, exports every declared entry point,
and rejects bad arguments on the host before any HIP call (no device needed)."""
import ctypes
import glob
import os
import re

import pytest

import tensor_head_attention_amd as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        txt = open(h).read()
        names += re.findall(r"^THA_API\s+[\w\s\*]*?\b(\w+)\s*\(", txt, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(T.LIB_PATH):
        import tensor_head_attention_amd.build as b
        b.build_library()
    return T.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_symbols()
    assert {"attn_fwd", "attn_fwd_ex", "attn_bwd", "attn_merge_lse", "shard_permute", "shard_unpermute",
            "tha_status_string", "tha_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert T.version() >= 101


def test_status_strings(lib):
    for s in (0, -1, -2, -3, 7):
        assert isinstance(T.status_string(s), str) and T.status_string(s)


def test_missing_library_fails_loudly(tmp_path):
    saved = T._lib
    try:
        T._lib = None
        with pytest.raises(RuntimeError):
            T.load_library(str(tmp_path / "nope.so"))
    finally:
        T._lib = saved


P = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails before any HIP call


def _attn(lib, q=P, k=P, v=P, o=P, out_dt=1, lse=None, B=1, Sq=8, Sk=8, H=1, D=128, in_dt=1, flags=0, qp=0, kp=0,
          kv=None, scale=0.088, stream=None):
    return lib.attn_fwd(q, k, v, o, out_dt, lse, B, Sq, Sk, H, D, in_dt, flags, qp, kp, kv, scale, stream)


def test_attn_fwd_validation(lib):
    E, U = T.THA_ERR_INVALID, T.THA_ERR_UNSUPPORTED
    assert _attn(lib, q=None) == E
    assert _attn(lib, k=None) == E
    assert _attn(lib, v=None) == E
    assert _attn(lib, o=None) == E
    for kw in ("B", "Sq", "Sk", "H", "D"):
        assert _attn(lib, **{kw: 0}) == E
        assert _attn(lib, **{kw: -3}) == E
    assert _attn(lib, flags=4) == E                      # unknown mask bit
    assert _attn(lib, flags=T.THA_MASK_KEY_PADDING) == E  # key padding without kv_len
    assert _attn(lib, scale=float("inf")) == E
    assert _attn(lib, scale=float("nan")) == E
    assert _attn(lib, scale=0.0) == E
    assert _attn(lib, scale=-0.5) == E
    assert _attn(lib, qp=1 << 62) == E
    assert _attn(lib, kp=-(1 << 62)) == E
    assert _attn(lib, in_dt=5) == U
    assert _attn(lib, out_dt=9) == U
    assert _attn(lib, D=96) == U                         # bf16 path: D in {64, 128}
    assert _attn(lib, in_dt=0, D=257) == U               # fp32 path: D <= 256
    assert _attn(lib, H=1 << 20, D=128) == U             # token row too long for 32-bit tile offsets
    assert _attn(lib, H=1 << 30, D=1 << 30, Sq=1 << 30) == U  # H*D*Sq far past 64 bits: rejected, no overflow


def _fwdx(lib, q=P, k=P, v=P, o=P, out_dt=1, lse=P, B=2, Sq=8, Sk=8, H=1, D=128, in_dt=1, flags=0, qp=0, kp=0,
          kv=None, scale=0.088, strides=None, stream=None):
    st = (ctypes.c_longlong * 8)(*strides) if strides is not None else None
    return lib.attn_fwd_ex(q, k, v, o, out_dt, lse, B, Sq, Sk, H, D, in_dt, flags, qp, kp, kv, scale, st, stream)


def test_attn_fwd_ex_validation(lib):
    E, U = T.THA_ERR_INVALID, T.THA_ERR_UNSUPPORTED
    hd = 128
    ok = [8 * 3 * hd, 3 * hd, 8 * 3 * hd, 3 * hd, 8 * 3 * hd, 3 * hd, 8 * hd, hd]  # packed QKV, contiguous o
    assert _attn(lib, flags=T.THA_ACCUMULATE) == E                         # attn_fwd has no accumulate mode
    assert _fwdx(lib, q=None, strides=ok) == E
    assert _fwdx(lib, flags=T.THA_ACCUMULATE, out_dt=1, strides=ok) == E   # accumulate needs an fp32 o
    assert _fwdx(lib, flags=T.THA_ACCUMULATE, out_dt=0, lse=None, strides=ok) == E  # ... and an lse
    assert _fwdx(lib, flags=64, strides=ok) == E                            # unknown flag bit
    assert _fwdx(lib, flags=5 << 3, strides=ok) == E                        # unknown kernel form
    assert _attn(lib, flags=T.THA_KERNEL_NARROW) == E                      # attn_fwd takes no kernel form
    for kf in (T.THA_KERNEL_NARROW, T.THA_KERNEL_WIDE, T.THA_KERNEL_SPLIT):  # valid forms pass to the next check
        assert _fwdx(lib, flags=kf, q=None, strides=ok) == E
    bad = list(ok); bad[1] = hd - 8                                         # token stride < H*D
    assert _fwdx(lib, strides=bad) == E
    bad = list(ok); bad[0] = 3 * hd                                         # batches overlap
    assert _fwdx(lib, strides=bad) == E
    bad = list(ok); bad[6] = -1
    assert _fwdx(lib, strides=bad) == E
    bad = list(ok); bad[4], bad[5] = 8 * 4 * hd, 4 * hd                     # k and v token strides differ
    assert _fwdx(lib, strides=bad) == U
    bad = list(ok); bad[0], bad[1] = 8 * (3 * hd + 4), 3 * hd + 4           # bf16 q stride not 16-byte aligned
    assert _fwdx(lib, strides=bad) == U
    assert _fwdx(lib, q=ctypes.c_void_p(0x1008), strides=ok) == U         # misaligned bf16 q
    bad = list(ok); bad[3] = bad[5] = 1 << 25                               # token stride too long
    assert _fwdx(lib, strides=bad) == E


def _bwd(lib, q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P, B=1, Sq=8, Sk=8, H=1, D=128, in_dt=1,
         flags=0, qp=0, kp=0, kv=None, scale=0.088, stream=None):
    return lib.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, Sq, Sk, H, D, in_dt, flags, qp, kp, kv, scale, stream)


def test_attn_bwd_validation(lib):
    E, U = T.THA_ERR_INVALID, T.THA_ERR_UNSUPPORTED
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"):
        assert _bwd(lib, **{name: None}) == E, name
    for kw in ("B", "Sq", "Sk", "H", "D"):
        assert _bwd(lib, **{kw: 0}) == E
    assert _bwd(lib, flags=4) == E
    assert _bwd(lib, flags=T.THA_MASK_KEY_PADDING) == E
    assert _bwd(lib, scale=float("nan")) == E
    assert _bwd(lib, scale=0.0) == E
    assert _bwd(lib, qp=1 << 62) == E
    assert _bwd(lib, in_dt=3) == U
    assert _bwd(lib, D=96) == U
    assert _bwd(lib, in_dt=0, D=300) == U
    assert _bwd(lib, H=1 << 20, D=128) == U
    for name in ("q", "k", "v", "do", "dq", "dk", "dv"):                  # bf16 path: 16-byte aligned vectors
        assert _bwd(lib, **{name: ctypes.c_void_p(0x1008)}) == U, name


def _ptr_arr(n, val=0x1000):
    return (ctypes.c_void_p * n)(*([val] * n))


def test_merge_validation(lib):
    E, U = T.THA_ERR_INVALID, T.THA_ERR_UNSUPPORTED
    o, l = _ptr_arr(2), _ptr_arr(2)
    ok = dict(n=2, o=o, l=l, pdt=0, out=P, odt=1, lo=None, B=1, S=4, H=2, D=8)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.attn_merge_lse(a["n"], a["o"], a["l"], a["pdt"], a["out"], a["odt"], a["lo"], a["B"], a["S"],
                                  a["H"], a["D"], None)
    assert call(n=0) == E
    assert call(n=65) == E
    assert call(o=None) == E
    assert call(l=None) == E
    assert call(out=None) == E
    assert call(o=(ctypes.c_void_p * 2)(0x1000, 0)) == E
    assert call(S=0) == E
    assert call(D=-1) == E
    assert call(pdt=3) == U
    assert call(odt=3) == U
    assert call(o=_ptr_arr(2, 0x2000), out=ctypes.c_void_p(0x2000), pdt=0, odt=1) == E  # in place, dtypes differ
    assert call(o=(ctypes.c_void_p * 2)(0x1000, 0x2000), out=ctypes.c_void_p(0x2000), pdt=1, odt=0) == E  # part 1


def test_permute_validation(lib):
    E, U = T.THA_ERR_INVALID, T.THA_ERR_UNSUPPORTED
    sh = _ptr_arr(4)
    for fn in (lambda *a: lib.shard_permute(a[0], a[1], a[2], a[3], *a[4:]),
               lambda *a: lib.shard_unpermute(a[3], a[1], a[2], a[0], *a[4:])):
        def call(shards=sh, Pn=4, g=0, out=P, B=1, S=8, H=8, D=4, eb=2):
            return fn(shards, Pn, g, out, B, S, H, D, eb, None)
        assert call(shards=None) == E
        assert call(out=None) == E
        assert call(Pn=0) == E
        assert call(Pn=65, shards=_ptr_arr(65)) == E
        assert call(g=4) == E
        assert call(g=-1) == E
        assert call(S=10) == E   # S % P
        assert call(H=6) == E    # H % P
        assert call(B=0) == E
        assert call(shards=(ctypes.c_void_p * 4)(0x1000, 0x1000, 0, 0x1000)) == E
        assert call(eb=3) == U


def test_all_to_all_validation(lib):
    E, U = T.THA_ERR_INVALID, T.THA_ERR_UNSUPPORTED
    ins = _ptr_arr(4)

    def call(inputs=ins, Pn=4, rank=0, out=P, shape=(2, 8, 8, 4), sd=2, gd=1, eb=2, nd=None):
        sh = (ctypes.c_longlong * len(shape))(*shape) if shape is not None else None
        return lib.shard_all_to_all(inputs, Pn, rank, out, len(shape) if nd is None else nd, sh, sd, gd, eb, None)
    assert call(inputs=None) == E
    assert call(out=None) == E
    assert call(shape=None, nd=4) == E
    assert call(Pn=0) == E
    assert call(Pn=65, inputs=_ptr_arr(65)) == E
    assert call(rank=4) == E
    assert call(rank=-1) == E
    assert call(nd=0) == E
    assert call(shape=(2,) * 9) == E            # more than 8 dims
    assert call(sd=1, gd=1) == E                # scatter dim == gather dim
    assert call(sd=4) == E
    assert call(gd=-1) == E
    assert call(shape=(2, 8, 6, 4)) == E        # 6 heads over 4 ranks
    assert call(shape=(2, 0, 8, 4)) == E        # empty dim
    assert call(shape=(1 << 25, 1 << 25, 8, 1)) == E  # more than 2^48 elements
    assert call(shape=(1 << 40, 1 << 40, 1 << 40, 4)) == E  # the product would overflow 64 bits
    assert call(inputs=(ctypes.c_void_p * 4)(0x1000, 0x1000, 0, 0x1000)) == E
    assert call(eb=3) == U


def test_attn_bwd_noalloc_validation(lib):
    """Every check of attn_bwd, then the scratch capacity, all on the host (no HIP call)."""
    E, U, L = T.THA_ERR_INVALID, T.THA_ERR_UNSUPPORTED, T.THA_ERR_TOO_LARGE

    def call(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, Sq=8, Sk=8, H=1, D=128, in_dt=1, flags=0,
             qp=0, kp=0, kv=None, scale=0.088):
        return lib.attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, Sq, Sk, H, D, in_dt, flags, qp, kp, kv,
                                    scale, None)
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert call(**{name: None}) == E, name
    assert call(B=0) == E
    assert call(flags=T.THA_MASK_KEY_PADDING) == E
    assert call(scale=-1.0) == E
    assert call(D=96) == U
    assert call(dq=ctypes.c_void_p(0x1008)) == U
    assert call(Sq=T.THA_NOALLOC_MAX_DELTA + 1) == L
    assert call(B=2, H=4, Sq=T.THA_NOALLOC_MAX_DELTA // 8 + 1) == L
    assert T.status_string(L)


def test_permute_n_validation(lib):
    E, U = T.THA_ERR_INVALID, T.THA_ERR_UNSUPPORTED
    for fn in (lib.shard_permute_n, lib.shard_unpermute_n):
        def call(n=3, Pn=4, sh=None, g=0, outs=None, B=1, S=8, H=8, D=4, eb=2):
            sh = _ptr_arr(n * Pn) if sh is None else sh
            outs = _ptr_arr(n) if outs is None else outs
            if fn is lib.shard_permute_n:
                return fn(n, sh, Pn, g, outs, B, S, H, D, eb, None)
            return fn(n, outs, Pn, g, sh, B, S, H, D, eb, None)
        assert call(n=0, sh=_ptr_arr(4), outs=_ptr_arr(1)) == E
        assert call(n=5) == E                                       # more than THA_MAX_PERMUTE_TENSORS
        assert call(outs=(ctypes.c_void_p * 3)(0x1000, 0, 0x1000)) == E
        bad = _ptr_arr(12)
        bad[7] = None                                               # tensor 1, shard 3
        assert call(sh=bad) == E
        assert call(g=4) == E
        assert call(S=10) == E
        assert call(H=6) == E
        assert call(eb=3) == U
