"""The balanced decode schedule's arithmetic, restated on the CPU.

The kernel deals the batch's 16-token tiles (sequences back to back) to NW
workgroups as [floor(w T / NW), floor((w + 1) T / NW)) with NW = min(nwc, T)
(nwc: 256 / unit chunks for 8-wave workgroups, 768 / unit chunks for the fp8
kernel's 4-wave ones), and gives piece k of sequence b the triple slot
owner(S_b) + b + k.  These checks hold that arithmetic to its invariants on
many length mixes and both grid sizes: every tile is covered once, the pieces
of a sequence go to consecutive workgroups with non-empty shares, and slots
are unique and below 768 + B (the workspace size pa_decode_plan reports)."""

import numpy as np
import pytest

TILE = 16
NWC = 256
SLOTS = 768   # shares per unit chunk the workspace holds slots for


def schedule(lengths, nwc=NWC):
    tiles = [(int(L) + TILE - 1) // TILE for L in lengths]
    S = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int64)
    T = int(S[-1])
    out = []  # (workgroup, b, first tile in b, end tile in b, slot or -1)
    if T == 0:
        return out, T, 0
    NW = min(nwc, T)

    def owner(t):
        return ((t + 1) * NW - 1) // T

    for wi in range(NW):
        tb, te = wi * T // NW, (wi + 1) * T // NW
        assert te > tb
        b = int(np.searchsorted(S[1:], tb, side="right"))
        while b < len(lengths) and S[b] < te:
            sb, se = int(S[b]), int(S[b + 1])
            if se > sb:
                first = owner(sb)
                pieces = owner(se - 1) - first + 1
                slot = first + b + (wi - first) if pieces > 1 else -1
                out.append((wi, b, max(tb, sb) - sb, min(te, se) - sb, slot))
            b += 1
    return out, T, NW


def _check(lengths, nwc=NWC):
    pieces, T, NW = schedule(lengths, nwc)
    B = len(lengths)
    covered = {}
    slots = set()
    by_seq = {}
    for wi, b, a, e, slot in pieces:
        assert 0 <= a < e
        for t in range(a, e):
            assert (b, t) not in covered
            covered[(b, t)] = wi
        by_seq.setdefault(b, []).append((wi, a, e, slot))
        if slot >= 0:
            assert slot not in slots
            assert 0 <= slot < SLOTS + B
            slots.add(slot)
    for b, L in enumerate(lengths):
        nt = (int(L) + TILE - 1) // TILE
        assert all((b, t) in covered for t in range(nt))
        ps = by_seq.get(b, [])
        assert len(ps) == (1 if nt else 0) or len(ps) > 1
        wis = [p[0] for p in ps]
        assert wis == list(range(wis[0], wis[0] + len(wis))) if wis else True
        if len(ps) > 1:
            assert [p[3] for p in ps] == list(range(ps[0][3], ps[0][3] + len(ps)))
            assert ps[0][1] == 0 and ps[-1][2] == nt
        elif len(ps) == 1:
            assert ps[0][3] == -1 and ps[0][1] == 0 and ps[0][2] == nt
    assert len(covered) == T


@pytest.mark.parametrize("nwc", [256, 64, 768, 384])
@pytest.mark.parametrize("seed", range(40))
def test_balanced_schedule_invariants(seed, nwc):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 3, 7, 31, 64, 255, 256, 257, 600, 2048]))
    kind = seed % 4
    if kind == 0:
        L = rng.integers(0, 40, B)              # fewer tiles than workgroups
    elif kind == 1:
        L = rng.integers(512, 2049, B)
    elif kind == 2:
        L = np.clip(np.rint(np.exp(rng.normal(7, 1, B))), 16, 16384)
    else:
        L = rng.integers(0, 3, B) * rng.integers(1, 5000, B)  # many zeros
    _check([int(x) for x in L], nwc)


def test_balanced_schedule_edges():
    _check([0])
    _check([0, 0, 0])
    _check([1])
    _check([16 * 256])          # exactly one tile per workgroup
    _check([16 * 256 + 1])
    _check([32768] * 4)
    _check([4096] * 64)         # every sequence in four pieces
