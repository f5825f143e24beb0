"""The decode's work split (walk_slice in decode.hip), modelled with the same
integer formulas on the CPU: the weighted positions (a tile counts kTileW,
each unit's start kSegW, tile j of a unit starting at kSegW + kTileW * j) cut
into slices of equal weight must give every tile of every unit to exactly one
slice, and the slices that walk one unit must be consecutive, each walking
at least one of its tiles, with the first one's split record naming the last
(the combine merges the partials of exactly those slices). The weights are
read from the kernel source."""

import os
import random
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "paged_kv_cache_316_amd", "csrc", "decode.hip")


def _weights():
    text = open(SRC).read()
    tw = int(re.search(r"constexpr int kTileW = (\d+);", text).group(1))
    sw = int(re.search(r"constexpr int kSegW = (\d+);", text).group(1))
    return tw, sw


def model(tiles_per_item, units, workers, TW, SW):
    S = len(tiles_per_item)
    total = sum(units * (TW * t + SW) for t in tiles_per_item if t > 0)
    W = min(total // TW, workers)
    unit_w = lambda n: TW * n + SW
    owner = {}          # (item, unit, tile) -> slice
    records = {}        # slice -> (item, unit, last_slice)
    slice_tiles = {}
    for w in range(workers):
        if w >= W:
            continue
        gb, ge = total * w // W, total * (w + 1) // W
        # locate
        pos = 0
        cur = None
        for s, t in enumerate(tiles_per_item):
            if t == 0:
                continue
            span = units * unit_w(t)
            if pos <= gb < pos + span:
                off = gb - pos
                u = off // unit_w(t)
                r = off - u * unit_w(t)
                j = 0 if r <= SW else (r - SW + TW - 1) // TW
                cur = dict(s=s, n=t, u=u, j=j, seg0=pos + u * unit_w(t))
                break
            pos += span
        assert cur is not None
        def advance():
            cur['j'] = 0
            cur['seg0'] += unit_w(cur['n'])
            cur['u'] += 1
            if cur['u'] == units:
                cur['u'] = 0
                while True:
                    cur['s'] += 1
                    cur['n'] = tiles_per_item[cur['s']] if cur['s'] < S else 0
                    if not (cur['n'] == 0 and cur['s'] + 1 < S):
                        break
        def tiles_before_end():
            room = ge - cur['seg0'] - SW
            return 0 if room <= 0 else min(cur['n'], (room + TW - 1) // TW)
        if cur['j'] >= cur['n']:
            advance()
        if tiles_before_end() <= cur['j']:
            continue
        cnt = 0
        while True:
            j1 = tiles_before_end()
            assert j1 > cur['j'], (w, cur, j1)
            assert cur['s'] < S and cur['n'] > 0
            for jj in range(cur['j'], j1):
                key = (cur['s'], cur['u'], jj)
                assert key not in owner, ("twice", key)
                owner[key] = w
                cnt += 1
            owns_start, owns_end = cur['j'] == 0, j1 == cur['n']
            if owns_start and not owns_end:
                last = cur['seg0'] + unit_w(cur['n']) - TW
                records[w] = (cur['s'], cur['u'], ((last + 1) * W - 1) // total)
            more = owns_end and cur['seg0'] + unit_w(cur['n']) + SW < ge
            if not more:
                break
            advance()
        slice_tiles[w] = cnt
    # every tile exactly once
    for s, t in enumerate(tiles_per_item):
        for u in range(units):
            for jj in range(t):
                assert (s, u, jj) in owner, ("missing", s, u, jj)
    # chains: a split segment's tiles are walked by consecutive slices [first, last], each non-empty
    for s, t in enumerate(tiles_per_item):
        for u in range(units):
            if t == 0:
                continue
            sl = sorted(set(owner[(s, u, jj)] for jj in range(t)))
            assert sl == list(range(sl[0], sl[-1] + 1)), ("gap", s, u, sl)
            if len(sl) > 1:
                assert records.get(sl[0], (None,))[:2] == (s, u), ("record", s, u, sl, records.get(sl[0]))
                assert records[sl[0]][2] == sl[-1], ("last", s, u, sl, records[sl[0]])
    return W, len(owner)



def test_kernel_weights_are_read():
    tw, sw = _weights()
    assert tw >= 1 and sw >= 0


@pytest.mark.parametrize("seed", range(6))
def test_every_tile_once_and_split_chains_contiguous(seed):
    tw, kernel_sw = _weights()
    rng = random.Random(seed)
    for _ in range(400):
        S = rng.randint(1, 40)
        tiles = [rng.choice([0, 1, 1, 2, 3, rng.randint(1, 40), rng.randint(1, 400)])
                 for _ in range(S)]
        if sum(tiles) == 0:
            continue
        units = rng.choice([1, 2, 4, 8, 40])
        workers = rng.choice([1, 2, 3, 5, 7, 16, 64, 300, 2048])
        sw = rng.choice([kernel_sw, 0, 1, 2, 3, 7])
        model(tiles, units, workers, tw, sw)
