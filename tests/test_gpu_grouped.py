"""GPU parity of pa_decode_grouped (the blocks a group of forked sequences
shares are read once per group) against the fp64 oracle, through the C ABI.

The parallel-sampling and beam-search workloads group their sequences as the
allocator forked them; the shared prefix of each group comes from the host
tables (pa_group_prefix_lens) and passes the precondition check. Synthetic
groups cover MHA and grouped heads (units of up to 16 columns, and groups
split into sub-groups), head_dim 64, blocks smaller and larger than a tile,
FP8 pools, empty tails, empty sequences, groups sharing nothing, prefixes
that differ between groups, and every split of the work between wavefronts.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_316_amd as pkv
import workloads
from oracle.attention import decode_attention
from oracle.expected import decode_out

from gpu_util import Loaded, assert_close, full_decode_out, full_workload, out_f64

pytestmark = pytest.mark.gpu

GROUP = {"cow": 3, "cow504": 3, "beam": 4}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def _grouped(g, wl, workers=0):
    M = GROUP[wl.name]
    tables, lens = g.tables.cpu().numpy(), g.lens.cpu().numpy()
    pl = pkv.group_prefix_lens(tables, lens, M, wl.block_size)
    pkv.check_grouped(g.pool, tables, lens, pl, M)
    out = torch.full_like(g.q, float("nan"))  # a row left unwritten shows up as NaN
    pkv.decode_grouped(g.q, g.pool, g.tables, g.lens, torch.from_numpy(pl).cuda(), M, wl.scale,
                       workers, out=out)
    torch.cuda.synchronize()
    return out, pl


@pytest.mark.parametrize("name", ["cow", "cow504", "beam"])
def test_sharing_workloads_small(name):
    wl = workloads.make(name, "small")
    g = Loaded(wl)
    out, pl = _grouped(g, wl)
    print(f"grouped: {name} small, prefix tokens per group {sorted(set(pl.tolist()))}", flush=True)
    assert (pl > 0).all(), "every group shares its prompt blocks"
    stats = assert_close(wl, out_f64(out), decode_out(wl), name)
    print(f"  {stats}", flush=True)


@pytest.mark.parametrize("name", ["cow", "beam"])
def test_default_work_slices(name):
    """Over bf16 pools the grouped decode defaults to 4 work slices per
    compute unit: a default call gives the same bits as one that asks for
    that count."""
    wl = workloads.make(name, "small")
    g = Loaded(wl)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    base, _ = _grouped(g, wl)
    explicit, _ = _grouped(g, wl, 4 * cus)
    assert torch.equal(base.view(torch.int16), explicit.view(torch.int16)), name


@pytest.mark.parametrize("workers", [1, 3, 7, 64, 333, 2048])
@pytest.mark.parametrize("name", ["cow504", "beam"])
def test_worker_splits(name, workers):
    """Units split between wavefronts at any tile (inside the shared prefix or
    inside a member's tokens) recombine by log-sum-exp to the oracle's result."""
    wl = workloads.make(name, "small")
    g = Loaded(wl)
    out, _ = _grouped(g, wl, workers)
    assert_close(wl, out_f64(out), decode_out(wl), f"{name} workers={workers}")


def _synthetic(Hq, Hkv, D, B, M, prefix_tokens, tails, dtype, seed, workers=0):
    """Groups of M sequences: group g shares prefix_tokens[g] tokens (whole
    blocks, written once) and member m then holds tails[g][m] tokens of its
    own. Blocks placed at random; every pool slot not written holds NaN."""
    rng = np.random.default_rng(seed)
    ng = len(prefix_tokens)
    S = ng * M
    nb_pre = [p // B for p in prefix_tokens]
    nb_tail = [[-(-t // B) for t in tails[g]] for g in range(ng)]
    total = sum(nb_pre) + sum(sum(x) for x in nb_tail)
    perm = rng.permutation(total + 4).astype(np.int32)
    lens = np.array([prefix_tokens[g] + tails[g][m] for g in range(ng) for m in range(M)], np.int32)
    maxb = max(1, max(-(-int(L) // B) for L in lens))
    tables = np.zeros((S, maxb), np.int32)
    io = torch.float32 if dtype == "f32" else torch.bfloat16
    ks, vs, slots, logical_k, logical_v = [], [], [], [], []
    nxt = 0

    def draw(n):
        return torch.from_numpy(rng.standard_normal((n, Hkv, D)).astype(np.float32)).to(io)

    for gi in range(ng):
        pre_blocks = perm[nxt:nxt + nb_pre[gi]]; nxt += nb_pre[gi]
        pk, pv = draw(prefix_tokens[gi]), draw(prefix_tokens[gi])
        t = np.arange(prefix_tokens[gi])
        if len(t):
            slots.append(pre_blocks[t // B].astype(np.int64) * B + t % B)
            ks.append(pk); vs.append(pv)
        for m in range(M):
            s = gi * M + m
            tb = perm[nxt:nxt + nb_tail[gi][m]]; nxt += nb_tail[gi][m]
            tables[s, :nb_pre[gi]] = pre_blocks
            tables[s, nb_pre[gi]:nb_pre[gi] + len(tb)] = tb
            tk, tv = draw(tails[gi][m]), draw(tails[gi][m])
            t = np.arange(tails[gi][m])
            if len(t):
                slots.append(tb[t // B].astype(np.int64) * B + t % B)
                ks.append(tk); vs.append(tv)
            logical_k.append(torch.cat([pk, tk])); logical_v.append(torch.cat([pv, tv]))
    if dtype == "fp8":
        ksc, vsc = 2.0 ** -6, 0.0123
        pool = pkv.KVPool.empty(total + 4, Hkv, B, D, torch.float8_e4m3fn, k_scale=ksc, v_scale=vsc)
        pool.k.view(torch.uint8).fill_(0x7F); pool.v.view(torch.uint8).fill_(0x7F)
    else:
        pool = pkv.KVPool.empty(total + 4, Hkv, B, D, io)
        pool.k.fill_(float("nan")); pool.v.fill_(float("nan"))
    if slots:
        pkv.cache_write(pool, torch.cat(ks).cuda(), torch.cat(vs).cuda(),
                        torch.from_numpy(np.concatenate(slots)).cuda())
    q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float32)).to(io)
    pl = np.repeat(np.asarray(prefix_tokens, np.int32), M)
    pkv.check_grouped(pool, tables, lens, pl, M)
    out = torch.full((S, Hq, D), float("nan"), dtype=io, device="cuda")  # unwritten rows: NaN
    pkv.decode_grouped(q.cuda(), pool, torch.from_numpy(tables).cuda(),
                       torch.from_numpy(lens).cuda(), torch.from_numpy(pl).cuda(), M,
                       1 / np.sqrt(D), workers, out=out)
    torch.cuda.synchronize()
    if dtype == "fp8":
        from oracle import fp8
        kk = [fp8.dequantize(fp8.quantize(k.float().numpy(), ksc), ksc) for k in logical_k]
        vv = [fp8.dequantize(fp8.quantize(v.float().numpy(), vsc), vsc) for v in logical_v]
    else:
        kk = [k.double().numpy() for k in logical_k]
        vv = [v.double().numpy() for v in logical_v]
    want = decode_attention(q.double().numpy(), kk, vv, 1 / np.sqrt(D))
    return out_f64(out), want, lens


class _Tol:
    dtype = "bf16"


CASES = {
    # name: (Hq, Hkv, D, B, M, prefix tokens per group, tails per group and member)
    "mha_m3": (4, 4, 128, 16, 3, [80, 160], [[0, 17, 40], [5, 1, 300]]),
    "gqa8_m2_16cols": (16, 2, 128, 16, 2, [96, 48, 512], [[3, 70], [0, 0], [129, 1]]),
    "gqa8_m4_subgroups": (16, 2, 128, 16, 4, [64, 32], [[9, 1, 33, 16], [2, 0, 45, 7]]),
    "gqa4_m4": (8, 2, 128, 16, 4, [208], [[31, 32, 33, 1]]),
    "d64_b8": (4, 2, 64, 8, 3, [40, 96], [[3, 11, 0], [64, 2, 9]]),
    "b4": (2, 2, 128, 4, 2, [12, 0], [[1, 30], [7, 5]]),
    "b32_no_sharing_group": (4, 4, 128, 32, 2, [0, 96], [[50, 70], [33, 0]]),
    "b64": (8, 8, 64, 64, 3, [128], [[1, 64, 200]]),
    "m1": (4, 4, 128, 16, 1, [32, 0, 48], [[5], [21], [0]]),
    "long_prefix": (4, 4, 128, 16, 3, [4096], [[1, 40, 600]]),
    "empty_member": (4, 4, 128, 16, 2, [0, 16], [[0, 33], [4, 7]]),
}


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", list(CASES))
def test_synthetic_groups(case, dtype):
    Hq, Hkv, D, B, M, pre, tails = CASES[case]
    got, want, lens = _synthetic(Hq, Hkv, D, B, M, pre, tails, dtype, seed=len(case) * 7 + M)
    stats = assert_close(_Tol, got, want, f"{case} {dtype}")
    print(f"grouped {case} {dtype}: {stats}", flush=True)
    for s in np.flatnonzero(lens == 0):  # a sequence without tokens: zeros
        assert np.all(got[s] == 0)


@pytest.mark.parametrize("workers", [1, 5, 29, 1000])
def test_synthetic_splits(workers):
    Hq, Hkv, D, B, M, pre, tails = CASES["gqa8_m2_16cols"]
    got, want, _ = _synthetic(Hq, Hkv, D, B, M, pre, tails, "bf16", seed=3, workers=workers)
    assert_close(_Tol, got, want, f"workers={workers}")


@pytest.mark.parametrize("workers", [8, 12, 100])
def test_columns_with_empty_partials(workers):
    """Regression: a group sharing nothing, split so that a wave sees only one
    member's tokens, leaves -inf partials for the other members' columns; two
    of them at the start of a merge must weigh 0, not turn the row into NaN."""
    got, want, _ = _synthetic(4, 4, 128, 32, 2, [0, 96], [[64, 64], [33, 0]], "bf16", seed=11,
                              workers=workers)
    assert_close(_Tol, got, want, f"workers={workers}")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["cow", "cow504", "beam"])
def test_sharing_workloads_full_every_row(name):
    """Full size, default launch configuration: every row against the oracle."""
    wl = full_workload(name)
    g = Loaded(wl)
    out, pl = _grouped(g, wl)
    print(f"grouped: {name} full, S={len(wl.decode_seqs)}, prefix tokens "
          f"{int(pl.min())}..{int(pl.max())}", flush=True)
    stats = assert_close(wl, out_f64(out), full_decode_out(name), f"{name} full")
    print(f"  all rows: {stats}", flush=True)
