"""CPU checks of the Python binding's argument validation: the C ABI sees raw pointers only, so
a tensor of the wrong shape, dtype or device must be rejected by the binding before any library
call.  The library is replaced by a recorder (no kernel runs; host tensors stand in for device
memory and are never dereferenced)."""
import pytest
import torch

import tensor_head_attention_amd as T


class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def rec(monkeypatch):
    r = _Recorder()
    monkeypatch.setattr(T, "_lib", r)
    monkeypatch.setattr(T, "_is_device", lambda t: True)
    monkeypatch.setattr(T, "_stream", lambda t: 0)
    return r


BF, F32 = torch.bfloat16, torch.float32


def _t(*shape, dtype=BF, device="cpu"):
    return torch.zeros(shape, dtype=dtype, device=device)


def _rejects(rec, fn, *a, **kw):
    with pytest.raises((ValueError, TypeError)):
        fn(*a, **kw)
    assert rec.calls == [], "the library was called despite a bad argument"


def test_attn_fwd_checks(rec):
    q, k, v = _t(2, 8, 3, 64), _t(2, 5, 3, 64), _t(2, 5, 3, 64)
    _rejects(rec, T.attn_fwd, q, _t(2, 5, 4, 64), v)                       # heads differ
    _rejects(rec, T.attn_fwd, q, _t(1, 5, 3, 64), _t(1, 5, 3, 64))         # batch differs
    _rejects(rec, T.attn_fwd, q, k, _t(2, 6, 3, 64))                       # v and k lengths differ
    _rejects(rec, T.attn_fwd, q, k, _t(2, 5, 3, 32))                       # head size differs
    _rejects(rec, T.attn_fwd, q, _t(2, 5, 3, 64, dtype=F32), v)            # dtypes differ
    _rejects(rec, T.attn_fwd, _t(8, 3, 64), k, v)                          # not 4-D
    _rejects(rec, T.attn_fwd, q, k, v, out=_t(2, 8, 3, 32))                # out shape
    _rejects(rec, T.attn_fwd, q, k, v, out=_t(2, 8, 3, 64, dtype=torch.float16))
    _rejects(rec, T.attn_fwd, q, k, v, lse=_t(2, 8, 3, dtype=F32))         # lse [B,H,Sq] expected
    _rejects(rec, T.attn_fwd, q, k, v, lse=_t(2, 3, 8, dtype=BF))          # lse dtype
    _rejects(rec, T.attn_fwd, q, k, v, kv_len=_t(3, dtype=torch.int32))    # kv_len length
    _rejects(rec, T.attn_fwd, q, k, v, kv_len=_t(2, dtype=torch.int64))    # kv_len dtype
    _rejects(rec, T.attn_fwd, q, _t(2, 5, 3, 64, device="meta"), v)        # another device
    _rejects(rec, T.attn_fwd, q, k, v, kernel="fast")                      # unknown kernel form
    T.attn_fwd(q, k, v, causal=True, kv_len=_t(2, dtype=torch.int32))
    T.attn_fwd(q, k, v, kernel="split")
    assert rec.calls == ["attn_fwd", "attn_fwd_ex"]


def test_attn_fwd_ex_checks(rec):
    qkv = _t(2, 8, 3, 4, 64)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    _rejects(rec, T.attn_fwd_ex, q, k[:, :, :3], v)                        # heads differ
    _rejects(rec, T.attn_fwd_ex, q, k, v[:, :5])                           # v and k lengths differ
    _rejects(rec, T.attn_fwd_ex, q, k, v, out=_t(2, 8, 4, 32))             # out shape
    _rejects(rec, T.attn_fwd_ex, q, k, v, lse=_t(2, 4, 7, dtype=F32))      # lse shape
    _rejects(rec, T.attn_fwd_ex, q, k, v, out=_t(2, 8, 4, 64, dtype=F32), lse=_t(2, 4, 8, dtype=F32),
             kv_len=_t(1, dtype=torch.int32))
    _rejects(rec, T.attn_fwd_ex, q, k, v, accumulate=True)                 # needs the running result
    T.attn_fwd_ex(q, k, v, out=_t(2, 8, 4, 64, dtype=F32), lse=_t(2, 4, 8, dtype=F32), accumulate=True)
    assert rec.calls == ["attn_fwd_ex"]


def test_attn_bwd_checks(rec):
    B, Sq, Sk, H, D = 2, 8, 5, 3, 64
    q, k, v = _t(B, Sq, H, D), _t(B, Sk, H, D), _t(B, Sk, H, D)
    o, do, lse = _t(B, Sq, H, D), _t(B, Sq, H, D), _t(B, H, Sq, dtype=F32)
    ok = dict(dq=_t(B, Sq, H, D, dtype=F32), dk=_t(B, Sk, H, D, dtype=F32), dv=_t(B, Sk, H, D, dtype=F32),
              workspace=_t(B * H * Sq, dtype=F32))
    _rejects(rec, T.attn_bwd, q, k, v, _t(B, Sk, H, D), do, lse, **ok)      # o shape
    _rejects(rec, T.attn_bwd, q, k, v, o, _t(B, Sq, H, D, dtype=F32), lse, **ok)  # dout dtype
    _rejects(rec, T.attn_bwd, q, k, v, o, do, _t(B, Sq, H, dtype=F32), **ok)  # lse layout
    _rejects(rec, T.attn_bwd, q, k, _t(B, Sk, H, 32), o, do, lse, **ok)     # v head size
    for name, bad in (("dq", _t(B, Sk, H, D, dtype=F32)), ("dk", _t(B, Sk, H, D)), ("dv", _t(B, Sq, H, D, dtype=F32)),
                      ("workspace", _t(B * H * Sq - 1, dtype=F32))):
        _rejects(rec, T.attn_bwd, q, k, v, o, do, lse, **dict(ok, **{name: bad}))
    _rejects(rec, T.attn_bwd, q, k, v, o, do, lse, kv_len=_t(B + 1, dtype=torch.int32), **ok)
    T.attn_bwd(q, k, v, o, do, lse, **ok)
    assert rec.calls == ["attn_bwd"]


def test_merge_checks(rec):
    B, S, H, D = 1, 6, 2, 16
    o = [_t(B, S, H, D, dtype=F32) for _ in range(3)]
    l = [_t(B, H, S, dtype=F32) for _ in range(3)]
    _rejects(rec, T.attn_merge_lse, o[:2] + [_t(B, S, H, 8, dtype=F32)], l)     # a part's shape
    _rejects(rec, T.attn_merge_lse, o[:2] + [_t(B, S, H, D)], l)                 # a part's dtype
    _rejects(rec, T.attn_merge_lse, o, l[:2] + [_t(B, S, H, dtype=F32)])         # an lse part's layout
    _rejects(rec, T.attn_merge_lse, o, l[:2])                                    # counts differ
    _rejects(rec, T.attn_merge_lse, o, l, out=_t(B, S, H, 8))                    # out shape
    _rejects(rec, T.attn_merge_lse, o, l, lse_out=_t(B, H, S + 1, dtype=F32))    # lse_out shape
    _rejects(rec, T.attn_merge_lse, [o[0]] * 65, [l[0]] * 65)                    # too many parts
    T.attn_merge_lse(o, l, out=o[2], lse_out=l[2])
    assert rec.calls == ["attn_merge_lse"]


def test_permute_checks(rec):
    P, B, Sl, H, D = 4, 1, 3, 8, 16
    sh = [_t(B, Sl, H, D) for _ in range(P)]
    _rejects(rec, T.shard_permute, sh[:3] + [_t(B, Sl + 1, H, D)], 0)            # shard shapes differ
    _rejects(rec, T.shard_permute, sh[:3] + [_t(B, Sl, H, D, dtype=F32)], 0)     # shard dtypes differ
    _rejects(rec, T.shard_permute, [_t(B, Sl, 6, D) for _ in range(P)], 0)       # heads not divisible
    _rejects(rec, T.shard_permute, sh, 0, out=_t(B, Sl * P, H, D))               # out shape
    _rejects(rec, T.shard_permute, sh, 0, out=_t(B, Sl * P, H // P, D, dtype=F32))
    x = _t(B, Sl * P, H // P, D)
    _rejects(rec, T.shard_unpermute, x, 0, [_t(B, Sl, H + 4, D) for _ in range(P)])  # shard heads
    _rejects(rec, T.shard_unpermute, _t(B, Sl * P + 1, H // P, D), 0, sh)           # sequence not divisible
    _rejects(rec, T.shard_unpermute, x, 0, sh[:3] + [_t(B, Sl, H, D, dtype=F32)])
    T.shard_permute(sh, 1)
    T.shard_unpermute(x, 1, sh)
    assert rec.calls == ["shard_permute", "shard_unpermute"]


def test_all_to_all_checks(rec):
    P = 4
    ins = [_t(2, 3, 8, 16) for _ in range(P)]
    _rejects(rec, T.shard_all_to_all, ins[:3] + [_t(2, 3, 8, 8)], 0, 2, 1)        # shapes differ
    _rejects(rec, T.shard_all_to_all, ins[:3] + [_t(2, 3, 8, 16, dtype=F32)], 0, 2, 1)  # dtypes differ
    _rejects(rec, T.shard_all_to_all, ins, 0, 1, 1)                                 # same dim twice
    _rejects(rec, T.shard_all_to_all, ins, 0, 4, 1)                                 # dim out of range
    _rejects(rec, T.shard_all_to_all, ins, 0, 1, 2)                                 # 3 tokens over 4 ranks
    _rejects(rec, T.shard_all_to_all, ins, 0, 2, 1, out=_t(2, 3, 2, 16))            # out shape
    _rejects(rec, T.shard_all_to_all, ins, 0, 2, 1, out=_t(2, 12, 2, 16, dtype=F32))
    T.shard_all_to_all(ins, 1, 2, 1)
    T.shard_all_to_all(ins, 1, -2, -3, out=_t(2, 12, 2, 16))
    assert rec.calls == ["shard_all_to_all", "shard_all_to_all"]


def test_permute_n_checks(rec):
    P, B, Sl, H, D = 4, 1, 3, 8, 16
    sets = [[_t(B, Sl, H, D) for _ in range(P)] for _ in range(3)]
    _rejects(rec, T.shard_permute_n, sets[:2] + [[_t(B, Sl, H, D) for _ in range(P - 1)]], 0)   # shard counts differ
    _rejects(rec, T.shard_permute_n, sets[:2] + [[_t(B, Sl + 1, H, D) for _ in range(P)]], 0)   # shapes differ
    _rejects(rec, T.shard_permute_n, sets + [sets[0], sets[1]], 0)                             # five tensors
    _rejects(rec, T.shard_permute_n, sets, 0, outs=[_t(B, Sl * P, H // P, D)] * 2)              # too few outputs
    _rejects(rec, T.shard_permute_n, sets, 0, outs=[_t(B, Sl * P, H, D)] * 3)                   # output shape
    xs = [_t(B, Sl * P, H // P, D) for _ in range(3)]
    _rejects(rec, T.shard_unpermute_n, xs, 0, sets[:2])                                        # sets != tensors
    _rejects(rec, T.shard_unpermute_n, xs[:2] + [_t(B, Sl * P, H // P, D, dtype=F32)], 0, sets)
    T.shard_permute_n(sets, 1)
    T.shard_unpermute_n(xs, 1, sets)
    assert rec.calls == ["shard_permute_n", "shard_unpermute_n"]


def test_kernel_names_map_to_flag_bits(monkeypatch):
    """kernel= reaches attn_fwd_ex as the THA_KERNEL_* bits of its flags (argument 12), next to the
    mask bits; no name means the automatic choice through attn_fwd."""
    seen = []

    class _Args:
        def __getattr__(self, name):
            def fn(*args):
                seen.append((name, args))
                return 0
            return fn
    monkeypatch.setattr(T, "_lib", _Args())
    monkeypatch.setattr(T, "_is_device", lambda t: True)
    monkeypatch.setattr(T, "_stream", lambda t: 0)
    q = _t(1, 8, 2, 128)
    names = {"narrow": T.THA_KERNEL_NARROW, "wide": T.THA_KERNEL_WIDE, "split": T.THA_KERNEL_SPLIT,
             "split64": T.THA_KERNEL_SPLIT64}
    assert len(set(names.values()) | {T.THA_KERNEL_AUTO}) == 5
    for name, bits in names.items():
        seen.clear()
        T.attn_fwd(q, q, q, causal=True, kernel=name)
        assert [n for n, _ in seen] == ["attn_fwd_ex"]
        assert seen[0][1][12] == T.THA_MASK_CAUSAL | bits, name
    for name in (None, "auto"):
        seen.clear()
        T.attn_fwd(q, q, q, causal=True, kernel=name)
        assert [n for n, _ in seen] == ["attn_fwd"] and seen[0][1][12] == T.THA_MASK_CAUSAL
