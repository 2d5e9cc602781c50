"""The balanced decode schedule's arithmetic, restated on the CPU.

The kernel deals the batch's 16-token tiles (sequences back to back) to NW
workgroups in equal ranges of cost, [floor(w T / NW), floor((w + 1) T / NW)).
A non-empty sequence costs its tiles plus K (the start of a piece, charged
as K tiles: positions S_b .. S_b + K - 1 are its start, its tiles follow),
and NW = min(nwc, T / (K + 1)) (nwc: 256 / unit chunks for 8-wave
workgroups, 768 / unit chunks for the fp8 kernel's 4-wave ones).  A tile
belongs to the share that holds its position, and piece k of sequence b gets
the triple slot owner(S_b + K) + b + k.  These checks hold that arithmetic to
its invariants on many length mixes, grid sizes and K (plain decode deals
with K = 0, the decode of the rest after a shared prefix with K = 3):
every tile is covered once, the pieces of a sequence go to consecutive
workgroups, every share holds a tile, and slots are unique and below
768 + B (the workspace size pa_decode_plan reports)."""

import numpy as np
import pytest

TILE = 16
NWC = 256
SLOTS = 768   # shares per unit chunk the workspace holds slots for
K_LIB = 3     # the shared-prefix decode's charge for a sequence start (plain decode: 0)


def schedule(lengths, nwc=NWC, K=K_LIB):
    tiles = [(int(L) + TILE - 1) // TILE for L in lengths]
    cost = [t + K if t else 0 for t in tiles]
    S = np.concatenate([[0], np.cumsum(cost)]).astype(np.int64)
    T = int(S[-1])
    out = []  # (workgroup, b, first tile in b, end tile in b, slot or -1)
    if T == 0:
        return out, T, 0
    NW = min(nwc, max(T // (K + 1), 1))

    def owner(t):
        return ((t + 1) * NW - 1) // T

    for wi in range(NW):
        tb, te = wi * T // NW, (wi + 1) * T // NW
        assert te > tb
        held = 0
        b = int(np.searchsorted(S[1:], tb, side="right"))
        while b < len(lengths) and S[b] < te:
            sb, se = int(S[b]), int(S[b + 1])
            r0 = sb + K
            a, e = max(tb, r0) - r0, min(te, se) - r0
            if se > sb and e > a:
                first = owner(r0)
                pieces = owner(se - 1) - first + 1
                slot = first + b + (wi - first) if pieces > 1 else -1
                out.append((wi, b, a, e, slot))
                held += e - a
            b += 1
        assert held > 0  # every share holds a tile
    return out, T, NW


def _check(lengths, nwc=NWC, K=K_LIB):
    pieces, T, NW = schedule(lengths, nwc, K)
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
    assert len(covered) == sum((int(L) + TILE - 1) // TILE for L in lengths)


@pytest.mark.parametrize("K", [0, K_LIB, 7])
@pytest.mark.parametrize("nwc", [256, 64, 768, 384])
@pytest.mark.parametrize("seed", range(40))
def test_balanced_schedule_invariants(seed, nwc, K):
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
    _check([int(x) for x in L], nwc, K)


@pytest.mark.parametrize("K", [0, K_LIB])
def test_balanced_schedule_edges(K):
    _check([0], K=K)
    _check([0, 0, 0], K=K)
    _check([1], K=K)
    _check([16 * 256], K=K)          # one tile per workgroup (K = 0)
    _check([16 * 256 + 1], K=K)
    _check([32768] * 4, K=K)
    _check([4096] * 64, K=K)         # every sequence in four pieces (K = 0)
    _check([16] * 2048, K=K)         # one tile each: K + 1 positions a sequence
    _check([16, 0, 5000, 17, 0, 0, 33] * 50, nwc=768, K=K)


def test_sequence_start_charge_evens_out_the_shares():
    """Shares that start more sequences hold fewer tiles: on a lognormal
    length mix, tiles + K x pieces spreads less across the shares than the
    tiles alone do with K = 0."""
    rng = np.random.default_rng(5)
    L = [int(x) for x in np.clip(np.rint(np.exp(rng.normal(7, 1, 128))), 16, 16384)]

    def spread(K):
        pieces, _, NW = schedule(L, 384, K)
        load = np.zeros(NW)
        for wi, b, a, e, slot in pieces:
            load[wi] += (e - a) + K_LIB  # time in tiles: a start costs about K_LIB
        return load.max() - load.mean()

    assert spread(K_LIB) < 0.6 * spread(0)


# --- shared-prefix decode: the grouped prefix work ---------------------------
#
# Below 1024 (sequence, query head) rows per kv head, pa_decode_shared_prefix
# adds grp_y rows of workgroups after the nwc decode shares of each unit
# chunk.  Wave gw of that part (workgroups in grid order, waves in
# workgroup order) takes piece gw // U of unit gw % U, U = Hkv * row_groups;
# a unit is (row group, kv head) with the kv head fastest, and column n of
# row group rg is row rg * 16 + n of the kv head's rows, sequence-major.  The
# prefix is cut into pieces of a multiple of 16 tokens, about 384 each.
# The decode shares give up the grouped rows of workgroups, so the grid is
# resident at once (at least a quarter of the shares stay).

GROUP_TOKENS = 384


def grouped_plan(B, Hq, Hkv, P, waves, chunks, workgroups):
    G = Hq // Hkv
    row_groups = (B * G + 15) // 16
    want = max(1, (P + GROUP_TOKENS - 1) // GROUP_TOKENS)
    tokens = ((P + want - 1) // want + 15) // 16 * 16
    pieces = (P + tokens - 1) // tokens
    units = Hkv * row_groups
    grp_y = ((units * pieces + waves - 1) // waves + chunks - 1) // chunks
    per = max(1, workgroups // chunks)
    nwc = max(per - grp_y, max(per // 4, 1))
    return dict(G=G, row_groups=row_groups, tokens=tokens, pieces=pieces, units=units,
                grp_y=grp_y, nwc=nwc)


def grouped_waves(B, Hq, Hkv, P, waves, chunks, workgroups):
    """(b, h, piece, token range, slot offset) for every live column of
    every grouped wave, as the kernel derives them."""
    pl = grouped_plan(B, Hq, Hkv, P, waves, chunks, workgroups)
    G, U = pl["G"], pl["units"]
    out = []
    for y in range(pl["nwc"], pl["nwc"] + pl["grp_y"]):
        for x in range(chunks):
            for w in range(waves):
                gw = ((y - pl["nwc"]) * chunks + x) * waves + w
                piece, unit = divmod(gw, U)
                if piece >= pl["pieces"]:
                    continue  # no unit: the wave exits
                kvh, rg = unit % Hkv, unit // Hkv
                lo = piece * pl["tokens"]
                hi = min(P, lo + pl["tokens"])
                for n in range(16):
                    r = rg * 16 + n
                    if r >= B * G:
                        continue
                    b, j = divmod(r, G)
                    out.append((b, kvh * G + j, piece, lo, hi, b * pl["pieces"] + piece))
    return out, pl


@pytest.mark.parametrize("B,Hq,Hkv,P,waves,chunks,workgroups", [
    (128, 32, 8, 1024, 4, 2, 768),   # the 1024-token fp8 prompt batch
    (40, 64, 8, 256, 8, 1, 256),     # bf16, group 8
    (5, 8, 8, 256, 8, 1, 256),       # MHA on the matrix-core path
    (4, 32, 8, 1200, 8, 1, 256),     # prefix not a multiple of 512
    (255, 16, 4, 96, 4, 1, 768),     # 1020 rows, one piece of 96
    (7, 96, 96, 2048, 8, 12, 256),   # many kv heads: a quarter of the shares stay
])
def test_grouped_prefix_work_covers_every_row_once(B, Hq, Hkv, P, waves, chunks, workgroups):
    cols, pl = grouped_waves(B, Hq, Hkv, P, waves, chunks, workgroups)
    assert B * (Hq // Hkv) < 1024
    seen = {}
    for b, h, piece, lo, hi, slot in cols:
        assert 0 <= b < B and 0 <= h < Hq and lo < hi <= P and lo % 16 == 0
        assert (b, h, piece) not in seen
        seen[(b, h, piece)] = (lo, hi)
        assert 0 <= slot < B * pl["pieces"]  # prefix slots follow the decode's
    assert len(seen) == B * Hq * pl["pieces"]
    for b in range(B):
        for h in range(Hq):
            ranges = sorted(seen[(b, h, k)] for k in range(pl["pieces"]))
            assert ranges[0][0] == 0 and ranges[-1][1] == P
            assert all(ranges[i][1] == ranges[i + 1][0] for i in range(len(ranges) - 1))
    # the decode shares and the grouped rows fit the grid and the workspace
    assert pl["nwc"] >= 1 and pl["nwc"] <= SLOTS and pl["nwc"] + pl["grp_y"] <= 65535
    assert pl["grp_y"] * chunks * waves >= pl["units"] * pl["pieces"]
    if pl["nwc"] > max(workgroups // chunks // 4, 1):
        assert (pl["nwc"] + pl["grp_y"]) * chunks <= workgroups  # one round
