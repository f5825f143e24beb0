"""pa_cache_write + pa_decode driven from a C program (tests/c/gpu_decode.c)
through the HIP runtime's C API: no Python or torch in the process that runs
the kernels. The test writes a seeded batch to raw files, runs the program on
the GPU and compares its output with the fp64 oracle."""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle.attention import decode_attention

from gpu_util import assert_close

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_cache_316_amd")


class _Bf16:
    dtype = "bf16"


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).bfloat16().view(torch.int16).numpy()


def _bf16_values(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    exe = tmp_path_factory.mktemp("cdrv") / "gpu_decode"
    cmd = ["gcc", "-std=gnu11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "gpu_decode.c"), "-L", PKG, "-l:libpagedkv.so",
           "-L/opt/rocm/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}", "-Wl,-rpath,/opt/rocm/lib",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (16, 2)])
def test_decode_from_c(driver, tmp_path, Hq, Hkv):
    D, B = 128, 16
    rng = np.random.default_rng(Hq * 10 + Hkv)
    lens = [1, 17, 100, 333, 64, 5]
    S = len(lens)
    nbs = [-(-L // B) for L in lens]
    nb = sum(nbs) + 4
    perm = rng.permutation(nb).astype(np.int32)
    maxb = max(nbs)
    tables = np.zeros((S, maxb), np.int32)
    at = 0
    for s, n in enumerate(nbs):
        tables[s, :n] = perm[at:at + n]
        at += n
    T = sum(lens)
    k_bits = _bf16_bits(rng.standard_normal((T, Hkv, D)))
    v_bits = _bf16_bits(rng.standard_normal((T, Hkv, D)))
    q_bits = _bf16_bits(rng.standard_normal((S, Hq, D)))
    slots = np.concatenate([tables[s, np.arange(L) // B].astype(np.int64) * B + np.arange(L) % B
                            for s, L in enumerate(lens)])
    scale = float(1 / np.sqrt(D))
    (tmp_path / "meta.txt").write_text(f"{S} {Hq} {Hkv} {D} {B} {nb} {maxb} {T} {scale!r}\n")
    k_bits.tofile(tmp_path / "k.bin")
    v_bits.tofile(tmp_path / "v.bin")
    slots.astype(np.int64).tofile(tmp_path / "slots.bin")
    q_bits.tofile(tmp_path / "q.bin")
    tables.tofile(tmp_path / "tables.bin")
    np.asarray(lens, np.int32).tofile(tmp_path / "lens.bin")
    print(f"C driver: Hq={Hq} Hkv={Hkv}, {S} sequences", flush=True)
    r = subprocess.run([str(driver), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got = _bf16_values(np.fromfile(tmp_path / "out.bin", dtype=np.int16).reshape(S, Hq, D))
    kv = _bf16_values(k_bits)
    vv = _bf16_values(v_bits)
    bounds = np.concatenate([[0], np.cumsum(lens)])
    want = decode_attention(_bf16_values(q_bits), [kv[bounds[s]:bounds[s + 1]] for s in range(S)],
                            [vv[bounds[s]:bounds[s + 1]] for s in range(S)], float(np.float32(scale)))
    print(f"  {assert_close(_Bf16, got, want, f'Hq={Hq} Hkv={Hkv}')}", flush=True)
