"""The C-ABI library on the CPU: it loads, exports every declared symbol,
rejects invalid requests before touching the device, and its host allocator
and block manager match the oracle's model operation by operation."""

import ctypes
import os
import re
import threading

import numpy as np
import pytest

from oracle.allocator import BadBlock, OutOfBlocks, RefCountAllocator, SequenceManager
from paged_kv_cache_462_amd import _lib
from paged_kv_cache_462_amd._lib import PaLaunch, PaTensor

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no binding signature"


def test_build_info():
    assert "gfx950" in _lib.load().pa_build_info().decode()


# --- validation without a device ---------------------------------------------

FAKE = 0x100000  # 16-byte aligned, never dereferenced: every case fails first


def _t(shape, dtype, stride=None, data=FAKE, scale=1.0):
    d = PaTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if stride is None:
        stride = []
        s = 1
        for x in reversed(shape):
            stride.insert(0, s)
            s *= x
    for i, (a, b) in enumerate(zip(shape, stride)):
        d.shape[i] = a
        d.stride[i] = b
    d.scale = scale
    return d


def _decode_args(B=2, Hq=8, Hkv=2, D=128, N=10, bs=16, mb=4, qdt=_lib.PA_BF16,
                 kvdt=_lib.PA_BF16, scale_k=1.0):
    return dict(out=_t([B, Hq, D], qdt), query=_t([B, Hq, D], qdt),
                kc=_t([N, bs, Hkv, D], kvdt, scale=scale_k),
                vc=_t([N, bs, Hkv, D], kvdt, scale=scale_k),
                tab=_t([B, mb], _lib.PA_I32), lens=_t([B], _lib.PA_I32),
                bs=bs, hkv=Hkv)


def _call_decode(a, launch=None, scale=0.1):
    lib = _lib.load()
    ln = launch if launch is not None else PaLaunch(None, None, 0, -1, 0)
    return lib.pa_decode(ctypes.byref(a["out"]), ctypes.byref(a["query"]), ctypes.byref(a["kc"]),
                         ctypes.byref(a["vc"]), ctypes.byref(a["tab"]), ctypes.byref(a["lens"]),
                         scale, a["bs"], a["hkv"], ctypes.byref(ln))


def _expect(rc, code):
    assert rc == code, (rc, _lib.last_error())
    assert _lib.last_error()


def test_decode_rejects_bad_group():
    a = _decode_args(Hq=6, Hkv=4)
    a["kc"] = _t([10, 16, 4, 128], _lib.PA_BF16)
    a["vc"] = _t([10, 16, 4, 128], _lib.PA_BF16)
    _expect(_call_decode(a), _lib.PA_ERR_INVALID_ARG)
    assert "multiple" in _lib.last_error()


@pytest.mark.parametrize("mut,code", [
    (lambda a: a.update(kc=_t([10, 16, 2, 96], _lib.PA_BF16), vc=_t([10, 16, 2, 96], _lib.PA_BF16),
                        out=_t([2, 8, 96], _lib.PA_BF16), query=_t([2, 8, 96], _lib.PA_BF16)),
     _lib.PA_ERR_UNSUPPORTED),
    (lambda a: a.update(kc=_t([10, 8, 2, 128], _lib.PA_BF16), vc=_t([10, 8, 2, 128], _lib.PA_BF16), bs=8),
     _lib.PA_ERR_UNSUPPORTED),
    (lambda a: a.update(bs=32), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(hkv=4), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(out=_t([2, 8, 128], _lib.PA_F16)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(kc=_t([10, 16, 2, 128], _lib.PA_F16), vc=_t([10, 16, 2, 128], _lib.PA_F16)),
     _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(query=_t([2, 8, 128], _lib.PA_BF16, data=0)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(query=_t([2, 8, 128], _lib.PA_BF16, data=FAKE + 2)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(kc=_t([10, 16, 2, 128], _lib.PA_BF16, stride=[4096, 256, 1, 2])),
     _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(tab=_t([2, 4], _lib.PA_I64)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(lens=_t([3], _lib.PA_I32)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(kc=_t([10, 16, 2, 128], _lib.PA_FP8_E4M3, scale=0.0),
                        vc=_t([10, 16, 2, 128], _lib.PA_FP8_E4M3, scale=0.0)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(out=_t([2, 8, 128], _lib.PA_F32), query=_t([2, 8, 128], _lib.PA_F32),
                        kc=_t([10, 16, 2, 128], _lib.PA_FP8_E4M3), vc=_t([10, 16, 2, 128], _lib.PA_FP8_E4M3)),
     _lib.PA_ERR_INVALID_ARG),
])
def test_decode_rejects(mut, code):
    a = _decode_args()
    mut(a)
    _expect(_call_decode(a), code)


def test_decode_table_reach_limit():
    # 2^26 blocks of 16 tokens address 2^30 token positions, the most a table
    # may reach; one block more is rejected (descriptors never dereferenced)
    a = _decode_args(B=1, mb=(1 << 26) + 1)
    _expect(_call_decode(a), _lib.PA_ERR_INVALID_ARG)
    assert "too many tokens" in _lib.last_error()
    # at the limit the call passes validation and, with the automatic plan
    # (which splits), stops at the missing workspace, before any launch
    a = _decode_args(B=1, mb=1 << 26)
    _expect(_call_decode(a, PaLaunch(None, None, 0, 0, 0)), _lib.PA_ERR_WORKSPACE)


def test_decode_needs_workspace_when_split():
    a = _decode_args(mb=64)  # 1024 tokens > 512-token partitions
    ln = PaLaunch(None, None, 0, 512, 0)
    _expect(_call_decode(a, ln), _lib.PA_ERR_WORKSPACE)
    need = _lib.load().pa_decode_workspace_bytes(2, 8, 2, 128, 16, 64, 512)
    assert need == 2 * 8 * 2 * (128 + 2) * 4
    ln = PaLaunch(None, FAKE, need - 4, 512, 0)
    _expect(_call_decode(a, ln), _lib.PA_ERR_WORKSPACE)


def test_decode_rejects_mfma_for_f32():
    a = _decode_args(qdt=_lib.PA_F32, kvdt=_lib.PA_F32)
    ln = PaLaunch(None, None, 0, -1, 2)
    _expect(_call_decode(a, ln), _lib.PA_ERR_UNSUPPORTED)


def _plan(*args):
    info = _lib.PaDecodePlan()
    rc = _lib.load().pa_decode_plan(*args, ctypes.byref(info))
    return rc, info


def test_plan():
    lib = _lib.load()
    B_ = _lib.PA_SCHEDULE_BALANCED
    # automatic: balanced shares of the batch's tiles
    rc, info = _plan(32, 32, 32, 128, 16, 128, 0)
    assert rc == 0 and info.schedule == B_ and info.partition_tokens == 0
    # shares per unit chunk the workspace holds: 768 (the fp8 kernel's grid
    # of 4-wave workgroups) + one per sequence
    slots = 768 + 32
    assert info.workspace_bytes == slots * 32 * 130 * 4 + 32 * 8
    assert lib.pa_decode_workspace_bytes(32, 32, 32, 128, 16, 128, 0) == info.workspace_bytes
    # automatic with a batch beyond the balanced limit: 512-token partitions
    rc, info = _plan(4096, 8, 8, 128, 16, 128, 0)
    assert rc == 0 and info.schedule == _lib.PA_SCHEDULE_PARTITIONS and info.partition_tokens == 512
    rc, info = _plan(4, 32, 8, 128, 16, 2048, -1)
    assert rc == 0 and info.schedule == _lib.PA_SCHEDULE_SINGLE and info.workspace_bytes == 0
    rc, info = _plan(4, 32, 8, 128, 16, 2048, 1024)
    assert rc == 0 and info.schedule == _lib.PA_SCHEDULE_PARTITIONS and info.partition_tokens == 1024
    rc, info = _plan(32, 32, 32, 128, 16, 32, 512)      # 512 tokens: one partition
    assert rc == 0 and info.schedule == _lib.PA_SCHEDULE_SINGLE
    # automatic with a table that reaches at most 256 tokens: one pass, no
    # workspace; one block more and the balanced schedule
    for mb, bs in ((16, 16), (7, 16), (8, 32), (0, 16)):
        rc, info = _plan(64, 32, 8, 128, bs, mb, 0)
        assert rc == 0 and info.schedule == _lib.PA_SCHEDULE_SINGLE and info.workspace_bytes == 0
        assert lib.pa_decode_workspace_bytes(64, 32, 8, 128, bs, mb, 0) == 0
    rc, info = _plan(64, 32, 8, 128, 16, 17, 0)
    assert rc == 0 and info.schedule == B_
    rc, _ = _plan(4, 32, 8, 128, 16, 2048, 100)
    assert rc == _lib.PA_ERR_INVALID_ARG
    assert lib.pa_decode_workspace_bytes(4, 32, 8, 128, 16, 2048, 512) == 4 * 32 * 64 * 130 * 4
    assert lib.pa_decode_workspace_bytes(4, 32, 8, 128, 16, 2048, -1) == 0
    assert lib.pa_decode_plan(4, 32, 8, 128, 16, 2048, 0, None) == _lib.PA_ERR_INVALID_ARG


def _cw_args(T=4, Hkv=2, D=128, N=10, bs=16, sdt=_lib.PA_BF16, cdt=_lib.PA_BF16, scale=1.0):
    return [_t([T, Hkv, D], sdt), _t([T, Hkv, D], sdt), _t([T], _lib.PA_I64),
            _t([N, bs, Hkv, D], cdt, scale=scale), _t([N, bs, Hkv, D], cdt, scale=scale)]


@pytest.mark.parametrize("mut,code", [
    (lambda a: a.__setitem__(2, _t([4], _lib.PA_I32)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.__setitem__(3, _t([10, 16, 2, 128], _lib.PA_F16)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.__setitem__(1, _t([4, 2, 128], _lib.PA_F16)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.__setitem__(0, _t([4, 2, 128], _lib.PA_BF16, stride=[256, 1, 2])), _lib.PA_ERR_INVALID_ARG),
    (lambda a: (a.__setitem__(3, _t([10, 16, 2, 128], _lib.PA_FP8_E4M3, scale=-1.0)),
                a.__setitem__(4, _t([10, 16, 2, 128], _lib.PA_FP8_E4M3, scale=-1.0))), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.__setitem__(0, _t([4, 2, 128], _lib.PA_I32)), _lib.PA_ERR_INVALID_ARG),
])
def test_cache_write_rejects(mut, code):
    a = _cw_args()
    mut(a)
    ln = PaLaunch(None, None, 0, 0, 0)
    rc = _lib.load().pa_reshape_and_cache(*(ctypes.byref(x) for x in a), ctypes.byref(ln))
    _expect(rc, code)


def test_cache_write_empty_is_noop():
    a = _cw_args(T=0)
    ln = PaLaunch(None, None, 0, 0, 0)
    assert _lib.load().pa_reshape_and_cache(*(ctypes.byref(x) for x in a), ctypes.byref(ln)) == 0


def _prefill_args(T=40, B=2, Hq=8, Hkv=2, D=128, N=10, bs=16, mb=4, qdt=_lib.PA_BF16,
                  kvdt=_lib.PA_BF16):
    return dict(out=_t([T, Hq, D], qdt), query=_t([T, Hq, D], qdt),
                kc=_t([N, bs, Hkv, D], kvdt), vc=_t([N, bs, Hkv, D], kvdt),
                tab=_t([B, mb], _lib.PA_I32), lens=_t([B], _lib.PA_I32),
                qsl=_t([B + 1], _lib.PA_I32), mq=0, bs=bs, hkv=Hkv)


def _call_prefill(a, scale=0.1):
    ln = PaLaunch(None, None, 0, 0, 0)
    return _lib.load().pa_prefill(
        ctypes.byref(a["out"]), ctypes.byref(a["query"]), ctypes.byref(a["kc"]),
        ctypes.byref(a["vc"]), ctypes.byref(a["tab"]), ctypes.byref(a["lens"]),
        ctypes.byref(a["qsl"]), a["mq"], scale, a["bs"], a["hkv"], ctypes.byref(ln))


@pytest.mark.parametrize("mut,code", [
    # head_dim 96 is not built
    (lambda a: a.update(kc=_t([10, 16, 2, 96], _lib.PA_BF16), vc=_t([10, 16, 2, 96], _lib.PA_BF16),
                        out=_t([40, 8, 96], _lib.PA_BF16), query=_t([40, 8, 96], _lib.PA_BF16)),
     _lib.PA_ERR_UNSUPPORTED),
    (lambda a: a.update(out=_t([40, 8, 128], _lib.PA_F32), query=_t([40, 8, 128], _lib.PA_F32),
                        kc=_t([10, 16, 2, 128], _lib.PA_F32), vc=_t([10, 16, 2, 128], _lib.PA_F32)),
     _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(qsl=_t([2], _lib.PA_I32)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(qsl=_t([3], _lib.PA_I64)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(tab=_t([3, 4], _lib.PA_I32)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(hkv=4), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(bs=32), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(kc=_t([10, 8, 2, 128], _lib.PA_BF16), vc=_t([10, 8, 2, 128], _lib.PA_BF16), bs=8),
     _lib.PA_ERR_UNSUPPORTED),
    (lambda a: a.update(kc=_t([10, 16, 2, 128], _lib.PA_F16), vc=_t([10, 16, 2, 128], _lib.PA_F16)),
     _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(out=_t([40, 8, 128], _lib.PA_BF16, data=FAKE + 8)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(query=_t([40, 8, 128], _lib.PA_BF16, stride=[1028, 128, 1])), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(out=_t([41, 8, 128], _lib.PA_BF16)), _lib.PA_ERR_INVALID_ARG),
    (lambda a: a.update(kc=_t([10, 16, 2, 128], _lib.PA_FP8_E4M3, scale=0.0),
                        vc=_t([10, 16, 2, 128], _lib.PA_FP8_E4M3, scale=0.0)), _lib.PA_ERR_INVALID_ARG),
])
def test_prefill_rejects(mut, code):
    a = _prefill_args()
    mut(a)
    _expect(_call_prefill(a), code)


def test_prefill_rejects_bad_group_and_scale():
    a = _prefill_args(Hq=6, Hkv=4)
    _expect(_call_prefill(a), _lib.PA_ERR_INVALID_ARG)
    _expect(_call_prefill(_prefill_args(), scale=float("inf")), _lib.PA_ERR_INVALID_ARG)
    _expect(_call_prefill(_prefill_args(), scale=0.0), _lib.PA_ERR_INVALID_ARG)
    _expect(_call_prefill(_prefill_args(), scale=-0.1), _lib.PA_ERR_INVALID_ARG)


def test_prefill_empty_is_noop():
    assert _call_prefill(_prefill_args(T=0)) == 0
    assert _call_prefill(_prefill_args(B=0)) == 0


def _call_shared(a, prefix, P, launch=None, scale=0.1):
    ln = launch if launch is not None else PaLaunch(None, FAKE, 1 << 40, 0, 0)
    return _lib.load().pa_decode_shared_prefix(
        ctypes.byref(a["out"]), ctypes.byref(a["query"]), ctypes.byref(a["kc"]),
        ctypes.byref(a["vc"]), ctypes.byref(a["tab"]), ctypes.byref(a["lens"]),
        ctypes.byref(prefix), P, scale, a["bs"], a["hkv"], ctypes.byref(ln))


def test_shared_prefix_rejects():
    a = _decode_args(mb=8)
    pb = _t([4], _lib.PA_I32)
    # f32 query; prefix not a multiple of the block size; prefix_blocks too
    # short or not int32; partitioning requested; negative scale
    f32 = _decode_args(qdt=_lib.PA_F32, kvdt=_lib.PA_F32, mb=8)
    _expect(_call_shared(f32, pb, 32), _lib.PA_ERR_INVALID_ARG)
    _expect(_call_shared(a, pb, 24), _lib.PA_ERR_INVALID_ARG)
    _expect(_call_shared(a, _t([1], _lib.PA_I32), 32), _lib.PA_ERR_INVALID_ARG)
    _expect(_call_shared(a, _t([4], _lib.PA_I64), 32), _lib.PA_ERR_INVALID_ARG)
    _expect(_call_shared(a, pb, 32, launch=PaLaunch(None, FAKE, 1 << 40, 512, 0)), _lib.PA_ERR_INVALID_ARG)
    _expect(_call_shared(a, pb, 32, scale=-1.0), _lib.PA_ERR_INVALID_ARG)
    # a prefix longer than the table addresses
    _expect(_call_shared(a, _t([16], _lib.PA_I32), 256), _lib.PA_ERR_INVALID_ARG)
    # workspace too small
    need = _lib.load().pa_decode_shared_prefix_workspace_bytes(2, 8, 2, 128, 16, 8, 32)
    _expect(_call_shared(a, pb, 32, launch=PaLaunch(None, FAKE, need - 16, 0, 0)), _lib.PA_ERR_WORKSPACE)
    # batches beyond the balanced schedule
    assert _lib.load().pa_decode_shared_prefix_workspace_bytes(4096, 8, 8, 128, 16, 8, 32) == \
        _lib.PA_ERR_UNSUPPORTED
    # below 1024 rows per kv head the grouped prefix work runs in the
    # matrix-core kernel: asking for the VALU path is refused
    _expect(_call_shared(a, pb, 32, launch=PaLaunch(None, FAKE, 1 << 40, 0, 1)), _lib.PA_ERR_UNSUPPORTED)
    assert "matrix-core" in _lib.last_error()


def test_shared_prefix_workspace_formula():
    lib = _lib.load()
    # fewer than 1024 (sequence, query head) rows per kv head: the grouped
    # prefix work, keys in pieces of about 384 (a multiple of 16), one
    # triple per (sequence, query head, piece) after the decode's own.
    # 128 x 4 rows, prefix 1024 -> 3 pieces of 352
    base = lib.pa_decode_workspace_bytes(128, 32, 8, 128, 32, 512, 0)
    got = lib.pa_decode_shared_prefix_workspace_bytes(128, 32, 8, 128, 32, 512, 1024)
    assert got == base + 128 * 3 * 32 * 130 * 4
    # prefix 96 -> one piece; prefix 1200 -> 4 pieces of 304 (the last 288)
    base = lib.pa_decode_workspace_bytes(3, 4, 2, 64, 16, 80, 0)
    assert lib.pa_decode_shared_prefix_workspace_bytes(3, 4, 2, 64, 16, 80, 96) == base + 3 * 1 * 4 * 66 * 4
    assert lib.pa_decode_shared_prefix_workspace_bytes(3, 4, 2, 64, 16, 80, 1200) == base + 3 * 4 * 4 * 66 * 4
    # 1024 rows or more: the prefix pass, 256-row tiles and enough pieces of
    # a multiple of 64 keys for about 256 workgroups.  200 x 8 rows: 7 row
    # tiles x 8 kv heads = 56 workgroups a piece -> 4 pieces of 128
    base = lib.pa_decode_workspace_bytes(200, 64, 8, 128, 16, 48, 0)
    got = lib.pa_decode_shared_prefix_workspace_bytes(200, 64, 8, 128, 16, 48, 512)
    assert got == base + 200 * 4 * 64 * 130 * 4
    # 256 x 4 rows = 1024: 4 row tiles x 8 = 32 a piece -> 8 pieces of 128
    base = lib.pa_decode_workspace_bytes(256, 32, 8, 128, 32, 512, 0)
    got = lib.pa_decode_shared_prefix_workspace_bytes(256, 32, 8, 128, 32, 512, 1024)
    assert got == base + 256 * 8 * 32 * 130 * 4


# --- allocator and block manager against the oracle's model ------------------

from paged_kv_cache_462_amd import BlockAllocator, BlockManager, PaError  # noqa: E402


def _code(fn, *a):
    try:
        return fn(*a), 0
    except PaError as e:
        return None, e.code
    except OutOfBlocks:
        return None, _lib.PA_ERR_OUT_OF_BLOCKS
    except BadBlock:
        return None, _lib.PA_ERR_BAD_BLOCK


def test_allocator_page_order_and_errors():
    a = BlockAllocator(4)
    assert [a.allocate() for _ in range(4)] == [3, 2, 1, 0]
    assert _code(a.allocate)[1] == _lib.PA_ERR_OUT_OF_BLOCKS
    a.decref(1)
    assert _code(a.decref, 1)[1] == _lib.PA_ERR_BAD_BLOCK
    assert _code(a.incref, 7)[1] == _lib.PA_ERR_BAD_BLOCK
    assert _code(a.incref, 1)[1] == _lib.PA_ERR_BAD_BLOCK
    assert a.allocate() == 1
    with pytest.raises(PaError):
        BlockAllocator(3, [0, 0, 1])


def test_allocator_matches_model_random():
    rng = np.random.default_rng(1)
    for trial in range(30):
        n = int(rng.integers(1, 40))
        order = rng.permutation(n).tolist() if trial % 2 else None
        ours, model = BlockAllocator(n, order), RefCountAllocator(n, order)
        for _ in range(300):
            op = int(rng.integers(0, 3))
            blk = int(rng.integers(-2, n + 2))
            if op == 0:
                r1, r2 = _code(ours.allocate), _code(model.allocate)
            elif op == 1:
                r1, r2 = _code(ours.incref, blk), _code(model.incref, blk)
            else:
                r1, r2 = _code(ours.decref, blk), _code(model.decref, blk)
            assert r1 == r2
            assert ours.num_free() == model.num_free()
        for b in range(n):
            assert ours.refcount(b) == model.refcount(b)


def test_block_manager_matches_model_random():
    rng = np.random.default_rng(2)
    for trial in range(20):
        n, bs = 48, int(rng.choice([1, 2, 4, 16]))
        ca, ma = BlockAllocator(n), RefCountAllocator(n)
        cm, mm = BlockManager(ca, bs), SequenceManager(ma, bs)
        live, nxt = [], 0
        for _ in range(300):
            op = int(rng.integers(0, 5))
            if op == 0 or not live:
                # sometimes attach a shared prefix of existing blocks
                shared, tok = [], 0
                if live and rng.random() < 0.5:
                    src = live[int(rng.integers(len(live)))]
                    tb = mm.tables[src]
                    k = int(rng.integers(0, len(tb) + 1))
                    shared = tb[:k]
                    tok = min(mm.lens[src], k * bs)
                r1 = _code(cm.add_sequence, nxt, shared, tok)
                r2 = _code(mm.add, nxt, shared, tok)
                assert r1[1] == r2[1]
                if r1[1] == 0:
                    live.append(nxt)
                nxt += 1
            elif op in (1, 2):
                s = live[int(rng.integers(len(live)))]
                r1, r2 = _code(cm.append_slot, s), _code(mm.append, s)
                assert r1 == (r2[0], r2[1]) if r2[1] == 0 else r1[1] == r2[1]
            elif op == 3:
                s = live[int(rng.integers(len(live)))]
                r1, r2 = _code(cm.fork, s, nxt), _code(mm.fork, s, nxt)
                assert r1[1] == r2[1]
                live.append(nxt)
                nxt += 1
            else:
                s = live.pop(int(rng.integers(len(live))))
                cm.free_sequence(s)
                mm.free(s)
            assert ca.num_free() == ma.num_free()
        if live:
            mb = max(len(t) for t in mm.tables.values()) + 1
            tables, lens = cm.export(live, mb)
            for i, s in enumerate(live):
                t = mm.tables[s]
                assert tables[i, :len(t)].tolist() == t and (tables[i, len(t):] == -1).all()
                assert lens[i] == mm.lens[s]
        for b in range(n):
            assert ca.refcount(b) == ma.refcount(b)


def test_block_manager_cow_pair():
    a = BlockAllocator(8)
    m = BlockManager(a, 4)
    m.add_sequence(0)
    for _ in range(6):
        m.append_slot(0)
    m.fork(0, 1)
    slot, src, dst = m.append_slot(1)
    assert (src, dst) == (6, 5) and slot == 22
    assert m.seq_len(1) == 7 and m.num_blocks_of(1) == 2
    with pytest.raises(PaError) as e:
        m.append_slot(99)
    assert e.value.code == _lib.PA_ERR_NOT_FOUND


def test_allocator_thread_hammer():
    """Concurrent allocate/decref from several threads (ctypes drops the GIL)."""
    a = BlockAllocator(256)
    errors = []

    def work(seed):
        rng = np.random.default_rng(seed)
        held = []
        try:
            for _ in range(4000):
                if held and (rng.random() < 0.5 or len(held) > 20):
                    a.decref(held.pop(int(rng.integers(len(held)))))
                else:
                    try:
                        held.append(a.allocate())
                    except PaError as e:
                        assert e.code == _lib.PA_ERR_OUT_OF_BLOCKS
            for b in held:
                a.decref(b)
        except Exception as e:  # pragma: no cover
            errors.append(e)

    th = [threading.Thread(target=work, args=(s,)) for s in range(8)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors
    assert a.num_free() == 256
    assert all(a.refcount(b) == 0 for b in range(256))


def test_prefill_workspace_bytes():
    """One int32 per workgroup of the prefill grid: query heads x query-tile
    ranks (256 rows each, from max_query_len, else the row count) x batch."""
    lib = _lib.load()
    assert lib.pa_prefill_workspace_bytes(8, 32, 16384, 2048) == 4 * 32 * 8 * 8
    assert lib.pa_prefill_workspace_bytes(4, 64, 4096, 1024) == 4 * 64 * 4 * 4
    assert lib.pa_prefill_workspace_bytes(4, 64, 4096, 0) == 4 * 64 * 16 * 4     # <= 0: the row count
    assert lib.pa_prefill_workspace_bytes(3, 8, 300, 257) == 4 * 8 * 2 * 3
    assert lib.pa_prefill_workspace_bytes(0, 8, 0, 0) == 0
    assert lib.pa_prefill_workspace_bytes(-1, 8, 10, 10) == _lib.PA_ERR_INVALID_ARG


def test_prefill_rejects_misaligned_workspace_and_flags():
    """Checked on the host, before any launch: a bf16 prefill's workspace
    (its f16-product flags) and any call's error flags must be 4-byte
    aligned."""
    a = _prefill_args()
    lib = _lib.load()

    def call(ln):
        return lib.pa_prefill(
            ctypes.byref(a["out"]), ctypes.byref(a["query"]), ctypes.byref(a["kc"]),
            ctypes.byref(a["vc"]), ctypes.byref(a["tab"]), ctypes.byref(a["lens"]),
            ctypes.byref(a["qsl"]), a["mq"], 0.1, a["bs"], a["hkv"], ctypes.byref(ln))

    _expect(call(PaLaunch(None, FAKE + 2, 1 << 20, 0, 0)), _lib.PA_ERR_INVALID_ARG)
    _expect(call(PaLaunch(None, None, 0, 0, 0, FAKE + 2)), _lib.PA_ERR_INVALID_ARG)
    cw = _cw_args()
    _expect(lib.pa_reshape_and_cache(*(ctypes.byref(x) for x in cw),
                                     ctypes.byref(PaLaunch(None, None, 0, 0, 0, FAKE + 2))),
            _lib.PA_ERR_INVALID_ARG)
