"""Pins of the oracle's block swap (CPU only): a hand-worked example whose
expected pools are written out element by element, the round trip out and
back in, and planted mistakes (source and destination exchanged, K and V
crossed, one head left behind) that the pins must catch."""

import numpy as np
import pytest

from oracle.paging import PoolMirror, swap

NAN16 = 0x7FC1


def _pool(nb, fill=None, seed=0):
    p = PoolMirror(nb, 2, 4, 8, np.uint16, NAN16)
    if fill == "iota":  # block b, head h, slot t, dim d holds b*1000 + h*100 + t*10 + d (+ 5000 in V)
        b, h, t, d = np.meshgrid(np.arange(nb), np.arange(2), np.arange(4), np.arange(8),
                                 indexing="ij")
        p.k[...] = b * 1000 + h * 100 + t * 10 + d
        p.v[...] = p.k + 5000
    elif fill == "random":
        rng = np.random.default_rng(seed)
        p.k[...] = rng.integers(0, 1 << 16, p.k.shape)
        p.v[...] = rng.integers(0, 1 << 16, p.v.shape)
    return p


def pin_hand_example(swap_fn):
    dev = _pool(3, "iota")
    host = _pool(4)
    swap_fn(host, dev, [(2, 0), (0, 3)])
    # host block 0 = device block 2, host block 3 = device block 0, blocks 1, 2 untouched
    assert host.k[0, 1, 3, 7] == 2000 + 100 + 30 + 7 and host.v[0, 1, 3, 7] == 7137
    assert host.k[3, 0, 2, 5] == 25 and host.v[3, 0, 2, 5] == 5025
    for b in (1, 2):
        assert (host.k[b] == NAN16).all() and (host.v[b] == NAN16).all()
    assert np.array_equal(host.k[0], dev.k[2]) and np.array_equal(host.k[3], dev.k[0])


def pin_round_trip(swap_fn):
    dev = _pool(6, "random", seed=1)
    orig_k, orig_v = dev.k.copy(), dev.v.copy()
    host = _pool(5)
    out = [(4, 0), (1, 2), (5, 4)]
    swap_fn(host, dev, out)
    dev.k[[4, 1, 5]] = NAN16  # the device blocks are reused meanwhile
    dev.v[[4, 1, 5]] = NAN16
    back = [(0, 3), (2, 0), (4, 5)]  # into other device blocks
    swap_fn(dev, host, back)
    assert np.array_equal(dev.k[3], orig_k[4]) and np.array_equal(dev.v[3], orig_v[4])
    assert np.array_equal(dev.k[0], orig_k[1]) and np.array_equal(dev.v[0], orig_v[1])
    assert np.array_equal(dev.k[5], orig_k[5]) and np.array_equal(dev.v[5], orig_v[5])
    assert np.array_equal(dev.k[2], orig_k[2])  # never a destination
    assert (dev.k[[1, 4]] == NAN16).all()


PINS = [pin_hand_example, pin_round_trip]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_swap_pins(pin):
    pin(swap)


def _swap_reversed(dst, src, pairs):
    swap(dst, src, [(d, s) for s, d in pairs])


def _swap_crossed(dst, src, pairs):
    for s, d in pairs:
        dst.k[d] = src.v[s]
        dst.v[d] = src.k[s]


def _swap_one_head(dst, src, pairs):
    for s, d in pairs:
        dst.k[d, 0] = src.k[s, 0]
        dst.v[d, 0] = src.v[s, 0]


@pytest.mark.parametrize("mutant", [_swap_reversed, _swap_crossed, _swap_one_head],
                         ids=lambda f: f.__name__)
def test_planted_swap_mistakes_are_caught(mutant):
    caught = 0
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, IndexError):
            caught += 1
    assert caught >= 1
