"""FP8 cache write, code by code: every bf16 bit pattern goes through
pa_cache_write into E4M3 pools and each stored byte is compared with the
oracle's quantize (IEEE fp32 division by the pool scale, saturation at +-448,
round to nearest even, NaN -> 0x7F).

The scale pairs cover the cases where the conversion can go wrong: a
power-of-two scale (exact division), a scale that makes x / scale round
(0.0123), a small scale under which most values saturate, and scales that
push quotients into fp32 subnormals (sign of zero results) or overflow.
Untouched slots must keep their fill byte.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_316_amd as pkv
from oracle import fp8

pytestmark = pytest.mark.gpu

D, HKV, B = 128, 1, 16
N_PAT = 1 << 16
T = N_PAT // (HKV * D)          # 512 token rows hold every pattern once
NUM_BLOCKS = 40                 # 640 slots, 128 of them left untouched
FILL = 0x55

SCALE_PAIRS = [
    (2.0 ** -6, 0.0123),
    (0.0123, 2.0 ** -6),
    (1e-3, 7.3),                # K: |x| > 0.448 saturates; V: many subnormal codes
    (1e37, 3.0e-38),            # K: quotients in fp32 subnormals; V: quotients overflow
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def _patterns():
    k_bits = np.arange(N_PAT, dtype=np.uint32).astype(np.uint16)
    v_bits = np.random.default_rng(11).permutation(k_bits)
    return k_bits, v_bits


@pytest.mark.parametrize("k_scale,v_scale", SCALE_PAIRS)
def test_every_bf16_pattern_codes_bit_exact(k_scale, v_scale):
    k_bits, v_bits = _patterns()
    slots = np.random.default_rng(12).choice(NUM_BLOCKS * B, size=T, replace=False).astype(np.int64)
    print(f"fp8 codes: k_scale={k_scale} v_scale={v_scale}, {N_PAT} patterns", flush=True)

    pool = pkv.KVPool.empty(NUM_BLOCKS, HKV, B, D, torch.float8_e4m3fn,
                            k_scale=k_scale, v_scale=v_scale)
    pool.k.view(torch.uint8).fill_(FILL)
    pool.v.view(torch.uint8).fill_(FILL)

    def dev(bits):
        t = torch.from_numpy(bits.view(np.int16).reshape(T, HKV, D).copy())
        return t.cuda().view(torch.bfloat16)

    pkv.cache_write(pool, dev(k_bits), dev(v_bits), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    got_k = pool.k.view(torch.uint8).cpu().numpy()
    got_v = pool.v.view(torch.uint8).cpu().numpy()

    # expected pool: fill byte everywhere, the oracle's codes at the written slots
    def expect(bits, scale):
        vals = (bits.astype(np.uint32) << 16).view(np.float32)  # bf16 -> fp32, exact
        codes = fp8.quantize(vals, scale).reshape(T, HKV, D)
        want = np.full((NUM_BLOCKS, HKV, B, D), FILL, dtype=np.uint8)
        want[slots // B, :, slots % B, :] = codes
        return want

    for name, got, bits, scale in (("K", got_k, k_bits, k_scale), ("V", got_v, v_bits, v_scale)):
        want = expect(bits, scale)
        bad = np.argwhere(got != want)
        if len(bad):
            b, h, o, d = bad[0]
            slot = b * B + o
            t = int(np.nonzero(slots == slot)[0][0]) if slot in slots else -1
            src = int(bits.reshape(T, HKV, D)[t, h, d]) if t >= 0 else -1
            pytest.fail(f"{name} scale={scale}: {len(bad)} bytes differ; first at block {b} "
                        f"offset {o} dim {d}: bf16 0x{src:04x} -> got 0x{got[b, h, o, d]:02x}, "
                        f"want 0x{want[b, h, o, d]:02x}")
