"""Pins for oracle.cache_write (O3): the page's append arithmetic and a
write / read-back round trip against the unpaged token stream."""

import numpy as np
import pytest
import torch

from oracle import cache_write as W
from oracle import fp8
from synth import get_config, make_workload
from synth.generate import empty_cache_cpu, shrink


def test_append_positions_follow_question_12():
    # sequence at length L appends into logical block L // bs, offset L % bs
    table = np.array([7, 3, 9, 2, 12])
    bs = 16
    for L in [0, 15, 16, 25, 67]:
        slot = table[L // bs] * bs + L % bs
        kc = torch.full((13, bs, 1, 2), float("nan"))
        vc = kc.clone()
        k = torch.tensor([[[1.5, -2.0]]])
        W.reshape_and_cache(k, k, np.array([slot]), kc, vc, "f32")
        assert torch.equal(kc[table[L // bs], L % bs, 0], k[0, 0])
        assert int(torch.isnan(kc).sum()) == 13 * bs * 2 - 2


@pytest.mark.parametrize("name", ["c1", "c2", "c5"])
def test_round_trip_small(name):
    cfg = shrink(get_config(name), batch=3, lengths=("list", [40, 1, 100]),
                 pool_blocks=0, pool_factor=1.5,
                 shared_prefix_tokens=32 if get_config(name).shared_prefix_tokens else 0)
    wl = make_workload(cfg, seed=5)
    kc = empty_cache_cpu(wl)
    vc = empty_cache_cpu(wl)
    kind = cfg.kv_dtype
    W.reshape_and_cache(wl.tok_key, wl.tok_value, wl.slot_mapping, kc, vc, kind,
                        wl.k_scale, wl.v_scale)
    # every written slot reads back the token (after the storage conversion)
    kf = W.to_f64(kc, kind, wl.k_scale)
    bs = cfg.block_size
    for i, s in enumerate(wl.slot_mapping):
        got = kf[s // bs, s % bs]
        src = wl.tok_key[i].to(torch.float32).numpy()
        if kind == "fp8":
            want = fp8.decode(fp8.quantize(src, wl.k_scale), wl.k_scale)
        else:
            want = src.astype(np.float64)
        assert np.array_equal(got, want)
    # slots nobody owns stay poisoned
    owned = np.zeros(wl.num_blocks * bs, bool)
    owned[wl.slot_mapping] = True
    flat = kf.reshape(wl.num_blocks * bs, -1)
    assert np.isnan(flat[~owned]).all()
    assert not np.isnan(flat[owned]).any()


def test_negative_slot_skips_and_duplicates_refused():
    kc = torch.zeros((2, 4, 1, 1))
    vc = torch.zeros((2, 4, 1, 1))
    k = torch.ones((3, 1, 1))
    W.reshape_and_cache(k, k, np.array([-1, 5, -7]), kc, vc, "f32")
    assert kc.sum() == 1 and kc[1, 1, 0, 0] == 1
    with pytest.raises(ValueError):
        W.reshape_and_cache(k, k, np.array([2, 2, 3]), kc, vc, "f32")


def test_bit_copy_keeps_nan_payloads():
    src = torch.tensor([0x7FC1, -1, 0x0001], dtype=torch.int16).view(torch.bfloat16).reshape(3, 1, 1)
    kc = torch.zeros((1, 4, 1, 1), dtype=torch.bfloat16)
    vc = kc.clone()
    W.reshape_and_cache(src, src, np.array([0, 1, 2]), kc, vc, "bf16")
    assert torch.equal(kc.view(torch.int16)[0, :3].flatten(), src.view(torch.int16).flatten())
