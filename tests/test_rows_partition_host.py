"""Host model of the whole-row decode's work partition and its merge (CPU only).

The decode kernel splits the tiles of all (batch, head group) sequences into
contiguous ranges of equal cost, one per workgroup: a sequence costs two steps
per valid 128-token block plus a start charge, and a tile goes to the range that
holds its cost midpoint.  A sequence whose tiles span several ranges is split:
each owner stores a partial in one of its two slots (slot 0 for the range's
first segment, slot 1 for its last) and tags the slot with the sequence.  The
merge kernel recomputes the first and last owners from the published partition
and reads the tags of the workgroups in between.  These tests check, over many
length mixes, that only a range's first and last segments are ever split, that
every tile has exactly one owner, and that the slots the merge finds are
exactly the ones the owners wrote.
"""
from __future__ import annotations

import random

import pytest

STEP_TOK = 128
SEG_W = 4                 # start charge of a sequence, in steps


def partition(seqs, ng, nblk, grid):
    """Units (v, t) -> owner, following the kernel's midpoint rule."""
    tile = nblk * STEP_TOK
    bv = len(seqs) * ng
    nbs = [(seqs[v // ng] + STEP_TOK - 1) // STEP_TOK for v in range(bv)]
    pref = [0]
    for nb in nbs:
        pref.append(pref[-1] + 2 * nb + (SEG_W if nb > 0 else 0))
    c = pref[-1]
    units = sum((seqs[v // ng] + tile - 1) // tile for v in range(bv))
    geff = min(grid, units)

    def mid(v, t):
        return pref[v] + (SEG_W // 2 if t == 0 else SEG_W) + 2 * nblk * t + min(nblk, nbs[v] - t * nblk)

    def lo(g):
        return g * c // geff

    def owner(x):
        return ((x + 1) * geff - 1) // c

    own = {}
    for v in range(bv):
        nt = (seqs[v // ng] + tile - 1) // tile
        for t in range(nt):
            m = mid(v, t)
            g = owner(m)
            assert lo(g) <= m < lo(g + 1) and 0 <= g < geff
            own[(v, t)] = g
    return dict(pref=pref, c=c, geff=geff, nbs=nbs, own=own, mid=mid, lo=lo, owner=owner, tile=tile)


def merger_list(part, v, nt, tags):
    """The slots the merge kernel reads for sequence v: owners g0..g1, by their tags."""
    mid, owner = part["mid"], part["owner"]
    g0, g1 = owner(mid(v, 0)), owner(mid(v, nt - 1))
    assert g1 - g0 + 1 <= 256
    out = []
    for g in range(g0, g1 + 1):
        if tags[2 * g] == v:
            out.append(2 * g)
        elif tags[2 * g + 1] == v:
            out.append(2 * g + 1)
    return out


def check(seqs, ng, nblk, grid):
    part = partition(seqs, ng, nblk, grid)
    if part["geff"] == 0:
        return 0
    tile = part["tile"]
    # each workgroup's units in order, its segments, and the tags it writes (a workgroup
    # with no unit writes -1 to both)
    by_g = {}
    for (v, t), g in sorted(part["own"].items()):
        by_g.setdefault(g, []).append((v, t))
    tags = [-1] * (2 * part["geff"])
    wrote = {}                                  # (v, g) -> (slot, tiles)
    for g, us in by_g.items():
        segs = []
        for v, t in us:
            if not segs or segs[-1][0] != v:
                segs.append([v, 0])
            segs[-1][1] += 1
        for i, (v, n) in enumerate(segs):
            nt = (seqs[v // ng] + tile - 1) // tile
            split = n != nt
            first, last = i == 0, i == len(segs) - 1
            if split:
                assert first or last, "only a range's first and last segments can be split"
                wrote[(v, g)] = (2 * g + (0 if first else 1), n)
            if first:
                tags[2 * g] = v if split else -1
            if last:
                tags[2 * g + 1] = v if (split and not first) else -1
    nsplit = 0
    for v in sorted({v for v, _ in wrote}):
        nt = (seqs[v // ng] + tile - 1) // tile
        owners = sorted(g for (vv, g) in wrote if vv == v)
        assert sum(wrote[(v, g)][1] for g in owners) == nt, "every tile is owned once"
        assert merger_list(part, v, nt, tags) == [wrote[(v, g)][0] for g in owners]
        nsplit += 1
    return nsplit


@pytest.mark.parametrize("seed", range(40))
def test_partition_and_merge_lists(seed):
    rng = random.Random(seed)
    ng = rng.choice([1, 2, 4])
    nblk = rng.choice([1, 2, 4, 8])
    b = rng.randint(1, 1024 // ng)
    kind = seed % 5
    if kind == 0:      # decode-like mix
        seqs = [rng.randint(1024, 8192) for _ in range(b)]
    elif kind == 1:    # a few very long sequences
        seqs = [rng.randint(65536, 131072) for _ in range(rng.randint(1, 4))]
    elif kind == 2:    # many short ones, some empty
        seqs = [rng.choice([0, 0, 1, 127, 128, 129, rng.randint(1, 2048)]) for _ in range(b)]
    elif kind == 3:    # one long among short ones
        seqs = [rng.randint(1, 300) for _ in range(b)]
        seqs[rng.randrange(b)] = 131072
    else:              # fewer units than workgroups
        seqs = [rng.randint(1, 3 * nblk * STEP_TOK) for _ in range(rng.randint(1, 12))]
    grid = rng.choice([256, 255, 80, 8, 1])
    check(seqs, ng, nblk, grid)


def test_narrow_ranges_hold_no_midpoint():
    """Ranges narrower than the tile spacing: some workgroups own no unit at all
    (and tag both slots -1), so the merge must skip them."""
    seqs = [65536] + [100] * 256                # 64 long tiles, then 256 one-block sequences
    assert check(seqs, 1, 8, 256) >= 1
    part = partition(seqs, 1, 8, 256)
    assert part["c"] // part["geff"] < 2 * 8     # ranges narrower than the tile spacing
    assert len(set(part["own"].values())) < part["geff"]


def test_headline_shape():
    rng = random.Random(1)
    seqs = [rng.randint(1024, 8192) for _ in range(32)]
    assert check(seqs, 4, 4, 256) > 100
