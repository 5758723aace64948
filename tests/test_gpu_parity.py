"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Small cases are compared element by element on every row; the full-size
workloads are compared on sampled rows the oracle computes one by one, plus
properties that hold at any size. Inputs come from the seeded generators in
`workloads`; the oracle reads host copies of the exact bytes the GPU used.
"""
import math
import os
import random

import pytest
import torch

import mla_ragged_chunked_amd as mra
import oracle
import workloads
from tests.parity import TOL, check, head_slice, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _flush(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    mra.lib()
    yield
    torch.cuda.synchronize()


def _to(x: workloads.PrefillInputs, device):
    return workloads.PrefillInputs(x.q.to(device), x.k.to(device), x.v.to(device), x.qo_indptr,
                                   x.kv_indptr, x.num_heads, x.causal, x.sm_scale)


def _full_parity(x: workloads.PrefillInputs, what):
    """Run on the GPU and compare every row with the oracle."""
    g = _to(x, DEV)
    _flush(f"[gpu] {what}: T={x.qo_indptr[-1]} Tk={x.kv_indptr[-1]} H={x.num_heads} "
           f"causal={x.causal} dtype={x.q.dtype}")
    o, lse = mra.ragged_prefill(g.q, g.k, g.v, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale)
    return check(o, lse, ro, rl, x.q.dtype, what)


# ---------------------------------------------------------------------------
# small workloads, every row
# ---------------------------------------------------------------------------

def test_tiny_fp32_workload():
    x = workloads.tiny_fp32()
    _full_parity(x, "tiny fp32 {1,17,64} x 4 heads")


@pytest.mark.parametrize("causal", [True, False])
def test_tiny_workload_in_bf16(causal):
    x = workloads.ragged_inputs([1, 17, 64], [1, 17, 64], 4, torch.bfloat16, seed=1,
                                causal=causal)
    _full_parity(x, f"tiny bf16 causal={causal}")


TILE_EDGE_LENS = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 513]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
def test_tile_edge_lengths(dtype, causal):
    x = workloads.ragged_inputs(TILE_EDGE_LENS, TILE_EDGE_LENS, 3, dtype, seed=31, causal=causal)
    _full_parity(x, f"tile edges dtype={dtype} causal={causal}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_qo_kv_mismatch_and_empty_sequences(dtype, causal):
    # qo > kv (causal rows with no key), kv = 0, qo = 0, kv > qo
    qo_lens = [5, 300, 0, 7, 513, 1, 260]
    kv_lens = [2, 0, 9, 40, 513, 700, 33]
    x = workloads.ragged_inputs(qo_lens, kv_lens, 2, dtype, seed=32, causal=causal)
    err = _full_parity(x, f"ragged mismatch dtype={dtype} causal={causal}")
    _flush(f"    max errors O={err[0]:.2e} LSE={err[1]:.2e}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
def test_single_head(dtype, causal):
    # H = 1: consecutive key rows are adjacent (384 B apart)
    lens = [1, 130, 33, 257]
    x = workloads.ragged_inputs(lens, [2 * n for n in lens], 1, dtype, seed=64, causal=causal)
    _full_parity(x, f"one head dtype={dtype} causal={causal}")


# bf16 plans pair two tiles of a sequence in one workgroup on batches of
# like sequences; each case below is such a batch
PAIRED_CASES = [
    # a full and a partial tile (22 rows: three of the four waves have no
    # row in it), causal and non-causal (non-causal: the partial tile first)
    ([150, 150, 140], [150, 150, 140], True),
    ([150, 150], [100, 120], False),
    # queries past the keys: pairs of tiles whose rows see no key
    ([280, 300], [3, 4], True),
    # a full tile paired with a tile of one or two rows
    ([129, 129, 130], [129, 129, 130], True),
    # non-causal sequences of >= 8 tiles over <= 4096 keys: all neighbours
    # pair (the last pair holds a 104-row tile)
    ([1000, 1000], [1500, 1400], False),
]


@pytest.mark.parametrize("case", range(len(PAIRED_CASES)))
def test_paired_workgroups_match_the_oracle(case):
    qo_lens, kv_lens, causal = PAIRED_CASES[case]
    x = workloads.ragged_inputs(qo_lens, kv_lens, 3, torch.bfloat16, seed=71 + case, causal=causal)
    plan = mra.Plan().plan(x.qo_indptr, x.kv_indptr, 3, causal, torch.bfloat16)
    assert plan.info()["items_per_workgroup"] == 2
    _full_parity(x, f"paired workgroups case {case}")


def _random_shape(rng):
    """A small random ragged batch: 1-6 sequences, lengths 0-600 (some empty),
    qo and kv drawn independently half of the time."""
    batch = int(rng.integers(1, 7))
    qo = [int(v) for v in rng.integers(0, 601, batch)]
    if rng.random() < 0.5:
        kv = list(qo)
    else:
        kv = [int(v) for v in rng.integers(0, 601, batch)]
    for i in range(batch):
        if rng.random() < 0.15:
            qo[i] = 0
        if rng.random() < 0.15:
            kv[i] = 0
    return qo, kv


@pytest.mark.parametrize("case", range(10))
def test_random_ragged_batches(case):
    import numpy as np
    rng = np.random.default_rng(1000 + case)
    qo, kv = _random_shape(rng)
    heads = int(rng.choice([1, 2, 3, 5, 8]))
    causal = bool(rng.random() < 0.6)
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    x = workloads.ragged_inputs(qo, kv, heads, dtype, seed=2000 + case, causal=causal)
    _full_parity(x, f"random case {case}: qo {qo} kv {kv} H={heads} causal={causal} {dtype}")


def test_more_than_128_heads():
    # H = 160: token rows 61,440 B apart, 32-bit per-lane offsets still small
    lens = [70, 1, 200]
    x = workloads.ragged_inputs(lens, lens, 160, torch.bfloat16, seed=65, causal=True)
    _full_parity(x, "160 heads")


def test_single_visible_key_is_exact_in_bf16():
    x = workloads.ragged_inputs([3, 300, 64], [3, 300, 64], 8, torch.bfloat16, seed=33)
    g = _to(x, DEV)
    o, lse = mra.ragged_prefill(g.q, g.k, g.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    torch.cuda.synchronize()
    for b in range(x.batch):
        t, j = x.qo_indptr[b], x.kv_indptr[b]
        # one visible key: p = 1, l = 1, so O is that V row bit for bit
        assert torch.equal(o[t].cpu(), x.v[j])
        s = (x.q[t].double() * x.k[j].double()).sum(-1) * x.sm_scale
        assert torch.allclose(lse[t].double().cpu(), s, atol=1e-5, rtol=0)


def test_equal_keys_average_visible_values_on_gpu():
    lens = [70, 300]
    x = workloads.ragged_inputs(lens, lens, 2, torch.bfloat16, seed=34)
    for b in range(x.batch):
        a, e = x.kv_indptr[b], x.kv_indptr[b + 1]
        x.k[a:e] = x.k[a:a + 1]
    _full_parity(x, "equal keys")


def test_more_heads_and_large_scores():
    # a large scale makes the running max move a lot (the lazy rescale path)
    lens = [400, 129]
    x = workloads.ragged_inputs(lens, lens, 5, torch.bfloat16, seed=35, sm_scale=0.5)
    _full_parity(x, "sm_scale 0.5")
    x = workloads.ragged_inputs(lens, lens, 5, torch.bfloat16, seed=36, sm_scale=1e-3)
    _full_parity(x, "sm_scale 1e-3")


def _rising_keys(k, kv_indptr, dim, step):
    """Key j of a sequence of L keys holds step * (j - (L - 1)) in `dim`
    (every head): rising scores that end near 0, so a row that sees the
    whole sequence has an LSE of a few units."""
    for b in range(len(kv_indptr) - 1):
        ks, ke = kv_indptr[b], kv_indptr[b + 1]
        j = torch.arange(ke - ks, dtype=torch.float64) - (ke - ks - 1)
        k[ks:ke, ..., dim] = (step * j).to(k.dtype).view(-1, *([1] * (k.dim() - 2)))


# fp32 only without the causal mask: early causal rows stop far below the
# last key, with LSEs of -75, where one fp32 ulp is near the 1e-5 tolerance
@pytest.mark.parametrize("dtype,causal", [(torch.bfloat16, True), (torch.bfloat16, False),
                                          (torch.float32, False)])
def test_running_max_rises_on_every_tile(dtype, causal):
    # Scores climb by ~8 (natural log units) per 32-key tile: every query
    # holds 1 in dim 0 and key j holds (j - last) / 4 there, the other query
    # dims are small noise. The running max then moves past the lazy
    # threshold on nearly every tile, so the O rescale runs on nearly every
    # tile.
    lens_q, lens_kv = [300, 129, 64, 1], [300, 129, 64, 700]
    x = workloads.ragged_inputs(lens_q, lens_kv, 3, dtype, seed=41, causal=causal, sm_scale=1.0)
    q, k = x.q.clone(), x.k.clone()
    q.mul_(0.05)
    q[..., 0] = 1.0
    _rising_keys(k, x.kv_indptr, 0, 0.25)
    x = workloads.PrefillInputs(q, k, x.v, x.qo_indptr, x.kv_indptr, x.num_heads, x.causal,
                                x.sm_scale)
    _full_parity(x, f"rising scores {dtype} causal={causal}")


@pytest.mark.parametrize("paired", [False, True])
def test_running_max_rises_paired_and_paged(paired):
    # The same forced rescale through the two-item kernel form (a batch of
    # like sequences, whose light tiles pair) or the one-item form, against
    # the oracle, and through the page pool, bit for bit against the
    # contiguous call (the paged kernels are separate instantiations).
    if paired:
        lens_q = lens_kv = [300, 260, 384]
    else:
        lens_q, lens_kv = [300, 129, 64, 1], [300, 129, 64, 700]
    x = workloads.ragged_inputs(lens_q, lens_kv, 3, torch.bfloat16, seed=47, causal=True,
                                sm_scale=1.0)
    q, k = x.q.clone(), x.k.clone()
    q.mul_(0.05)
    q[..., 0] = 1.0
    _rising_keys(k, x.kv_indptr, 0, 0.25)
    x = workloads.PrefillInputs(q, k, x.v, x.qo_indptr, x.kv_indptr, x.num_heads, x.causal,
                                x.sm_scale)
    plan = mra.Plan().plan(x.qo_indptr, x.kv_indptr, 3, True, torch.bfloat16)
    assert plan.info()["items_per_workgroup"] == (2 if paired else 1)
    _full_parity(x, f"rising scores paired={paired}")
    g = _to(x, DEV)
    kc, vc, table = _paged_cache(g, 64, extra_pages=2, seed=5)
    ref_o, ref_l = mra.ragged_prefill(g.q, g.k, g.v, x.qo_indptr, x.kv_indptr, True, 1.0)
    o, l = mra.ragged_prefill_paged(g.q, kc, vc, x.qo_indptr, x.kv_indptr, table, True, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_plan_run_matches_one_shot_and_repeats():
    lens = [300, 1, 129]
    x = _to(workloads.ragged_inputs(lens, lens, 4, torch.bfloat16, seed=37), DEV)
    o1, l1 = mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    for n_xcd in (8, 1):
        p = mra.Plan(n_xcd=n_xcd).plan(x.qo_indptr, x.kv_indptr, 4, True).upload()
        for _ in range(3):
            o2, l2 = p.run(x.q, x.k, x.v, x.sm_scale)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # without LSE
    o3 = mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale,
                            return_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)


HEAD_BLOCK_QO = [1, 31, 33, 64, 129, 300, 5, 0, 7, 260]
HEAD_BLOCK_KV = [1, 31, 33, 64, 129, 300, 2, 9, 0, 700]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
def test_head_blocks_match_the_oracle_and_single_heads(dtype, causal):
    # items that run 2, 4 or 8 heads back to back, across short, tile-edge,
    # empty and key-less sequences (the K/V ring runs on across heads)
    x = workloads.ragged_inputs(HEAD_BLOCK_QO, HEAD_BLOCK_KV, 8, dtype, seed=39, causal=causal)
    g = _to(x, DEV)
    _flush(f"[gpu] head blocks dtype={dtype} causal={causal}")
    ro, rl = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale)
    base = None
    for hpi in (1, 2, 4, 8):
        p = mra.Plan(heads_per_item=hpi).plan(x.qo_indptr, x.kv_indptr, 8, causal, dtype).upload()
        assert p.info()["heads_per_item"] == hpi
        o, lse = p.run(g.q, g.k, g.v, x.sm_scale)
        torch.cuda.synchronize()
        check(o, lse, ro, rl, dtype, f"head blocks of {hpi}")
        # each head runs the same arithmetic whatever the block size
        if base is None:
            base = (o, lse)
        else:
            assert torch.equal(o, base[0]) and torch.equal(lse, base[1])


DEVICE_PLAN_CASES = [
    ([5, 300, 0, 7, 513, 1, 260], [2, 0, 9, 40, 513, 700, 33], 3),
    ([1, 31, 33, 64, 129, 300], [1, 31, 33, 64, 129, 300], 16),
    ([128] * 9, [1000] * 9, 8),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("case", range(len(DEVICE_PLAN_CASES)))
def test_device_plan_matches_host_plan(dtype, causal, case):
    qo_lens, kv_lens, heads = DEVICE_PLAN_CASES[case]
    x = _to(workloads.ragged_inputs(qo_lens, kv_lens, heads, dtype, seed=40 + case, causal=causal),
            DEV)
    _flush(f"[gpu] device plan case {case} dtype={dtype} causal={causal}")
    ref_o, ref_l = mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    tq, tk = x.qo_indptr[-1], x.kv_indptr[-1]
    dp = mra.DevicePlan(len(qo_lens), tq, tk, heads, dtype)
    qo_d = torch.tensor(x.qo_indptr, dtype=torch.int32, device=DEV)
    kv_d = torch.tensor(x.kv_indptr, dtype=torch.int32, device=DEV)
    o, l = dp.run(x.q, x.k, x.v, qo_d, kv_d, causal, x.sm_scale)
    torch.cuda.synchronize()
    assert int(dp.invalid_flag().item()) == 0
    # same arithmetic per (row, head); only the order of work differs
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_device_plan_flags_invalid_indptrs_and_skips_them():
    lens = [40, 70, 90]
    x = _to(workloads.ragged_inputs(lens, lens, 4, torch.bfloat16, seed=43), DEV)
    tq = x.qo_indptr[-1]
    dp = mra.DevicePlan(3, tq, tq, 4)
    # sequence 1 ends beyond max_tq: skipped; sequences 0 and 2 stay in bounds
    bad = [0, 40, tq + 500, tq]
    assert all(0 <= a <= tq for a in (bad[0], bad[1], bad[3]))
    qo_d = torch.tensor(bad, dtype=torch.int32, device=DEV)
    out = torch.zeros((tq, 4, 128), dtype=torch.bfloat16, device=DEV)
    o, l = dp.run(x.q, x.k, x.v, qo_d, qo_d, True, x.sm_scale, out=out)
    torch.cuda.synchronize()
    assert int(dp.invalid_flag().item()) != 0
    ref_o, ref_l = mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    assert torch.equal(o[:40], ref_o[:40]) and torch.equal(l[:40], ref_l[:40])


def test_device_plan_in_a_captured_graph_follows_new_indptrs():
    # one captured graph (device plan + prefill), replayed after the indptr
    # contents change; every replay is checked against the eager host path
    heads, batch, max_t = 4, 4, 1024
    g = torch.Generator().manual_seed(44)
    q = workloads.randn((max_t, heads, 192), g, torch.bfloat16, "cpu").to(DEV)
    k = workloads.randn((max_t, heads, 192), g, torch.bfloat16, "cpu").to(DEV)
    v = workloads.randn((max_t, heads, 128), g, torch.bfloat16, "cpu").to(DEV)
    scale = 192 ** -0.5
    qo_d = torch.zeros(batch + 1, dtype=torch.int32, device=DEV)
    kv_d = torch.zeros(batch + 1, dtype=torch.int32, device=DEV)
    out = torch.zeros((max_t, heads, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((max_t, heads), dtype=torch.float32, device=DEV)
    dp = mra.DevicePlan(batch, max_t, max_t, heads)
    first = workloads.indptr_from_lengths([100, 200, 300, 400])
    qo_d.copy_(torch.tensor(first, dtype=torch.int32))
    kv_d.copy_(torch.tensor(first, dtype=torch.int32))
    dp.run(q, k, v, qo_d, kv_d, True, scale, out=out, lse=lse)      # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dp.run(q, k, v, qo_d, kv_d, True, scale, out=out, lse=lse)
    torch.cuda.synchronize()
    for lens in ([100, 200, 300, 400], [1, 513, 0, 300], [256, 256, 256, 256], [17, 4, 900, 33]):
        ind = workloads.indptr_from_lengths(lens)
        qo_d.copy_(torch.tensor(ind, dtype=torch.int32))
        kv_d.copy_(torch.tensor(ind, dtype=torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        t = ind[-1]
        ref_o, ref_l = mra.ragged_prefill(q[:t].contiguous(), k[:t].contiguous(), v[:t].contiguous(),
                                          ind, ind, True, scale)
        torch.cuda.synchronize()
        _flush(f"[gpu] graph replay lens={lens}")
        assert torch.equal(out[:t], ref_o) and torch.equal(lse[:t], ref_l)
        assert int(dp.invalid_flag().item()) == 0


def _paged_cache(x: workloads.PrefillInputs, page: int, extra_pages: int, seed: int):
    """Scatter the contiguous K/V of `x` into page-organised caches in a random
    page order (plus unused pages of finite filler) and return the caches and
    the block table."""
    g = torch.Generator().manual_seed(seed)
    lens = [b - a for a, b in zip(x.kv_indptr, x.kv_indptr[1:])]
    per = [-(-n // page) for n in lens]
    total = sum(per) + extra_pages
    h = x.k.shape[1]
    perm = torch.randperm(total, generator=g).tolist()
    kc = workloads.randn((total, page, h, 192), g, x.k.dtype, "cpu")
    vc = workloads.randn((total, page, h, 128), g, x.v.dtype, "cpu")
    table = torch.full((len(lens), max(max(per), 1)), -1, dtype=torch.int32)
    k_host, v_host = x.k.cpu(), x.v.cpu()
    i = 0
    for b, n in enumerate(lens):
        for pg in range(per[b]):
            phys = perm[i]
            i += 1
            table[b, pg] = phys
            a = x.kv_indptr[b] + pg * page
            m = min(page, n - pg * page)
            kc[phys, :m] = k_host[a:a + m]
            vc[phys, :m] = v_host[a:a + m]
    return kc.to(DEV), vc.to(DEV), table.to(DEV)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("page", [32, 64, 128])
def test_paged_kv_matches_contiguous(dtype, causal, page):
    qo_lens = [5, 300, 0, 7, 513, 1, 260]
    kv_lens = [2, 0, 9, 40, 513, 700, 33]
    x = _to(workloads.ragged_inputs(qo_lens, kv_lens, 3, dtype, seed=45, causal=causal), DEV)
    _flush(f"[gpu] paged page={page} dtype={dtype} causal={causal}")
    kc, vc, table = _paged_cache(x, page, extra_pages=5, seed=page)
    ref_o, ref_l = mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    o, l = mra.ragged_prefill_paged(x.q, kc, vc, x.qo_indptr, x.kv_indptr, table, causal,
                                    x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_paged_context_pass_against_the_oracle():
    # a chunked-prefill context pass (non-causal over a paged prefix) checked
    # directly against the oracle on the contiguous bytes
    qo_lens, kv_lens = [64, 1, 130], [200, 96, 257]
    x = workloads.ragged_inputs(qo_lens, kv_lens, 2, torch.bfloat16, seed=46, causal=False)
    g = _to(x, DEV)
    kc, vc, table = _paged_cache(g, 64, extra_pages=3, seed=7)
    o, l = mra.ragged_prefill_paged(g.q, kc, vc, x.qo_indptr, x.kv_indptr, table, False,
                                    x.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, False, x.sm_scale)
    check(o, l, ro, rl, torch.bfloat16, "paged context pass")


@pytest.mark.parametrize("case", range(8))
def test_entry_points_agree_on_random_batches(case):
    # Every route into the prefill on the same random ragged batch: the
    # one-shot call (checked against the oracle), a plan with 2-head items,
    # a page pool through a block table and the device-planned call. The
    # arithmetic per (row, head) is the same in all of them, so their
    # outputs must equal the one-shot call's bit for bit.
    import numpy as np
    rng = np.random.default_rng(3000 + case)
    qo, kv = _random_shape(rng)
    heads = int(rng.choice([2, 4, 6]))
    causal = bool(rng.random() < 0.6)
    dtype = torch.float32 if case % 4 == 3 else torch.bfloat16
    page = int(rng.choice([32, 64]))
    x = workloads.ragged_inputs(qo, kv, heads, dtype, seed=4000 + case, causal=causal)
    _flush(f"[gpu] entry points case {case}: qo {qo} kv {kv} H={heads} causal={causal} "
           f"{dtype} page={page}")
    g = _to(x, DEV)
    ref_o, ref_l = mra.ragged_prefill(g.q, g.k, g.v, x.qo_indptr, x.kv_indptr, causal,
                                      x.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    check(ref_o, ref_l, ro, rl, dtype, f"entry points case {case}")
    p = mra.Plan(heads_per_item=2).plan(x.qo_indptr, x.kv_indptr, heads, causal, dtype).upload()
    o, l = p.run(g.q, g.k, g.v, x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l), "2-head items"
    kc, vc, table = _paged_cache(g, page, extra_pages=2, seed=case)
    o, l = mra.ragged_prefill_paged(g.q, kc, vc, x.qo_indptr, x.kv_indptr, table, causal,
                                    x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l), "paged"
    tq, tk = x.qo_indptr[-1], x.kv_indptr[-1]
    dp = mra.DevicePlan(len(qo), max(tq, 1), max(tk, 1), heads, dtype)
    qo_d = torch.tensor(x.qo_indptr, dtype=torch.int32, device=DEV)
    kv_d = torch.tensor(x.kv_indptr, dtype=torch.int32, device=DEV)
    o, l = dp.run(g.q, g.k, g.v, qo_d, kv_d, causal, x.sm_scale)
    torch.cuda.synchronize()
    assert int(dp.invalid_flag().item()) == 0
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l), "device plan"


def test_one_shot_on_two_streams():
    lens = [200, 90]
    x = _to(workloads.ragged_inputs(lens, lens, 2, torch.bfloat16, seed=38), DEV)
    ref, ref_l = mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for s in (s1, s2, s1, s2):
        with torch.cuda.stream(s):
            outs.append(mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True,
                                           x.sm_scale))
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o, ref) and torch.equal(l, ref_l)


def test_one_shot_threads_sharing_a_stream():
    """Threads that enqueue one-shot calls on one stream take turns on its
    plan: every result equals the same call made alone."""
    import threading
    cases = [_to(workloads.ragged_inputs(lens, lens, 2, torch.bfloat16, seed=60 + i), DEV)
             for i, lens in enumerate(([300, 17], [64] * 5, [1, 2, 700], [129, 255, 33, 8]))]
    refs = []
    for x in cases:
        refs.append(mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    results = [[] for _ in cases]
    errors = []

    def work(i):
        try:
            x = cases[i]
            with torch.cuda.stream(stream):
                for _ in range(6):
                    results[i].append(mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr,
                                                         True, x.sm_scale))
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    _flush("[gpu] one-shot prefill from 4 threads on one stream")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (ro, rl), outs in zip(refs, results):
        assert len(outs) == 6
        for o, l in outs:
            assert torch.equal(o, ro) and torch.equal(l, rl)


def test_native_library_is_loaded():
    with open("/proc/self/maps") as fh:
        maps = fh.read()
    assert os.path.realpath(mra.LIB_PATH) in maps


# ---------------------------------------------------------------------------
# merge_state
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_merge_state_parity(dtype):
    o_a, l_a, o_b, l_b = workloads.merge_inputs(3000, 8, dtype, seed=41, neg_inf_frac=0.2)
    g = [t.to(DEV) for t in (o_a, l_a, o_b, l_b)]
    o, l = mra.merge_state(*g)
    torch.cuda.synchronize()
    ro, rl = oracle.merge(o_a, l_a, o_b, l_b)
    check(o, l, ro, rl, dtype, f"merge {dtype}")


def test_merge_state_beyond_one_pass():
    # More rows than one pass of the merge grid covers (2^20 workgroups of
    # 256 lanes at 16 lanes per bf16 row: 2^24 rows, i.e. 131072 tokens of
    # 128 heads), so the grid-stride loop runs; rows of both passes, some
    # with an empty side, are checked against the oracle.
    heads = 128
    tokens = (1 << 24) // heads + 64
    _flush(f"[gpu] merge_state beyond one pass: {tokens} tokens x {heads} heads")
    o_a, l_a, o_b, l_b = workloads.merge_inputs(tokens, heads, torch.bfloat16, seed=44, device=DEV,
                                                neg_inf_frac=0.05)
    o, l = mra.merge_state(o_a, l_a, o_b, l_b)
    torch.cuda.synchronize()
    rng = random.Random(9)
    pick = {0, 1, tokens // 2, (1 << 24) // heads - 1} | set(range(tokens - 64, tokens))
    pick |= {rng.randrange(tokens) for _ in range(64)}
    idx = torch.tensor(sorted(pick), device=DEV)
    ro, rl = oracle.merge(o_a[idx].cpu(), l_a[idx].cpu(), o_b[idx].cpu(), l_b[idx].cpu())
    check(o[idx], l[idx], ro, rl, torch.bfloat16, "merge beyond one pass")
    del o_a, l_a, o_b, l_b, o, l
    torch.cuda.empty_cache()


def test_merge_state_in_place():
    o_a, l_a, o_b, l_b = [t.to(DEV) for t in
                          workloads.merge_inputs(777, 4, torch.bfloat16, seed=42, neg_inf_frac=0.1)]
    ref_o, ref_l = mra.merge_state(o_a, l_a, o_b, l_b)
    mra.merge_state(o_a, l_a, o_b, l_b, out=o_a, out_lse=l_a)
    torch.cuda.synchronize()
    assert torch.equal(o_a, ref_o) and torch.equal(l_a, ref_l)


# ---------------------------------------------------------------------------
# decompression
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("num_seqs,seq_len,num_heads", [
    (2, 300, 3), (1, 17, 1), (3, 129, 4),
    (1, 4113, 16),   # many 32-token tiles per workgroup, a ragged last tile, empty token ranges
    (1, 33, 128),    # 128 heads, two tiles (the second holds one token)
    (2, 500, 5)])
def test_decompress_small_parity(num_seqs, seq_len, num_heads):
    # ragged token tails (not multiples of the 32-token tile), odd head counts
    d = workloads.decompress_batch(num_seqs=num_seqs, seq_len=seq_len, num_heads=num_heads)
    _flush(f"[gpu] decompress T={num_seqs * seq_len} H={num_heads}")
    k, v = mra.decompress_kv(d.c_kv.to(DEV), d.k_rope.to(DEV), d.w_uk.to(DEV), d.w_uv.to(DEV),
                             num_heads)
    torch.cuda.synchronize()
    rk, rv = oracle.decompress(d.c_kv, d.k_rope, d.w_uk, d.w_uv, num_heads)
    k, v = k.double().cpu(), v.double().cpu()
    # k_rope is copied, not computed
    assert torch.equal(k[:, :, 128:], rk[:, :, 128:])
    # bf16 output rounding (half an ulp, 2^-9 relative) plus fp32 accumulation
    for got, want in ((k[:, :, :128], rk[:, :, :128]), (v, rv)):
        err = (got - want).abs()
        assert torch.all(err <= want.abs() * 2.0 ** -8 + 1e-4), err.max()


# ---------------------------------------------------------------------------
# full-size workloads, sampled rows
# ---------------------------------------------------------------------------

def _sampled_parity(g: workloads.PrefillInputs, o, lse, heads, rows, what, q_host=None,
                    k_host=None, v_host=None):
    """Compare sampled rows of heads `heads` with the oracle (per-head host copies)."""
    for h in heads:
        qh = head_slice(g.q, h) if q_host is None else q_host(h)
        kh = head_slice(g.k, h) if k_host is None else k_host(h)
        vh = head_slice(g.v, h) if v_host is None else v_host(h)
        ro, rl = oracle.prefill(qh, kh, vh, g.qo_indptr, g.kv_indptr, g.causal, g.sm_scale,
                                rows)
        idx = torch.tensor(rows)
        check(o[idx, h:h + 1].cpu(), lse[idx, h:h + 1].cpu(), ro, rl,
              g.q.dtype if q_host is None else torch.bfloat16, f"{what} head {h}")


def _row_properties(o, lse):
    assert torch.isfinite(o).all(), "non-finite O"
    assert torch.isfinite(lse).all(), "non-finite LSE (every row sees a key here)"


def test_deepseek_v3_batch_full_size():
    g = workloads.deepseek_v3_batch(device=DEV)
    _flush(f"[gpu] deepseek_v3_batch T={g.qo_indptr[-1]} lens={g.qo_indptr}")
    o, lse = mra.ragged_prefill(g.q, g.k, g.v, g.qo_indptr, g.kv_indptr, True, g.sm_scale)
    torch.cuda.synchronize()
    _row_properties(o, lse)
    # both sides of every 128-row query-tile edge, sequence ends, random rows
    rows = sample_rows(g.qo_indptr, block=mra.PREFILL_BLOCK_M, n_random=128, seed=2)
    _sampled_parity(g, o, lse, [0, 41, 77, 127], rows, "deepseek_v3_batch")


def test_chunked_prefill_full_size():
    c = workloads.chunked_prefill(device=DEV)
    m = c.main
    _flush(f"[gpu] chunked_prefill: {len(c.chunks)} context chunks")
    parts = [mra.ragged_prefill(ch.q, ch.k, ch.v, ch.qo_indptr, ch.kv_indptr, False, ch.sm_scale)
             for ch in c.chunks]
    parts.append(mra.ragged_prefill(m.q, m.k, m.v, m.qo_indptr, m.kv_indptr, True, m.sm_scale))
    o, lse = parts[0]
    for o2, l2 in parts[1:]:
        o, lse = mra.merge_state(o, lse, o2, l2)
    torch.cuda.synchronize()
    _row_properties(o, lse)
    rows = sample_rows(m.qo_indptr, block=mra.PREFILL_BLOCK_M, n_random=64, seed=3)
    idx = torch.tensor(rows)
    for h in (0, 57, 101, 127):
        q = head_slice(m.q, h)
        chunk_kvs = [(head_slice(ch.k, h), head_slice(ch.v, h), ch.kv_indptr) for ch in c.chunks]
        ro, rl, rparts = oracle.chunked(q, head_slice(m.k, h), head_slice(m.v, h), m.qo_indptr,
                                        chunk_kvs, m.sm_scale, rows)
        for (po, pl), (qo_, ql_) in zip(parts, rparts):
            check(po[idx, h:h + 1].cpu(), pl[idx, h:h + 1].cpu(), qo_, ql_, torch.bfloat16,
                  f"chunked partial head {h}")
        check(o[idx, h:h + 1].cpu(), lse[idx, h:h + 1].cpu(), ro, rl, torch.bfloat16,
              f"chunked merged head {h}")


def test_skewed_batch_full_size():
    g = workloads.skewed_batch(device=DEV)
    _flush(f"[gpu] skewed_batch T={g.qo_indptr[-1]} max_len="
           f"{max(b - a for a, b in zip(g.qo_indptr, g.qo_indptr[1:]))}")
    o, lse = mra.ragged_prefill(g.q, g.k, g.v, g.qo_indptr, g.kv_indptr, True, g.sm_scale)
    torch.cuda.synchronize()
    _row_properties(o, lse)
    # every tile-edge row (both sides of each 128-row edge) and both ends of
    # every sequence, including the longest ones, plus random rows
    rows = sample_rows(g.qo_indptr, block=mra.PREFILL_BLOCK_M, n_random=64, seed=4)
    _flush(f"[gpu] skewed_batch: {len(rows)} sampled rows x 4 heads against the oracle")
    _sampled_parity(g, o, lse, [0, 5, 64, 127], rows, "skewed_batch")
    del g, o, lse
    torch.cuda.empty_cache()


def test_decompress_then_prefill_full_size():
    d = workloads.decompress_batch(device=DEV)
    H = d.num_heads
    _flush(f"[gpu] decompress_batch T={d.indptr[-1]} H={H}")
    k, v = mra.decompress_kv(d.c_kv, d.k_rope, d.w_uk, d.w_uv, H)
    o, lse = mra.ragged_prefill(d.q, k, v, d.indptr, d.indptr, True, d.sm_scale)
    torch.cuda.synchronize()
    _row_properties(o, lse)
    c_kv, k_rope = d.c_kv.cpu(), d.k_rope.cpu()
    rows = sample_rows(d.indptr, block=mra.PREFILL_BLOCK_M, n_random=32, seed=5)
    idx = torch.tensor(rows)
    for h in (0, 3, H - 2, H - 1):
        wk = d.w_uk[:, h * 128:(h + 1) * 128].contiguous().cpu()
        wv = d.w_uv[:, h * 128:(h + 1) * 128].contiguous().cpu()
        rk, rv = oracle.decompress(c_kv, k_rope, wk, wv, 1)           # fp64, all tokens
        # decompressed K/V for this head, sampled tokens: bf16 rounding bound
        gk = k[idx, h:h + 1].double().cpu()
        gv = v[idx, h:h + 1].double().cpu()
        assert torch.all((gk - rk[idx]).abs() <= rk[idx].abs() * 2.0 ** -8 + 1e-4)
        assert torch.all((gv - rv[idx]).abs() <= rv[idx].abs() * 2.0 ** -8 + 1e-4)
        qh = head_slice(d.q, h).double()
        ro, rl = oracle.prefill(qh, rk, rv, d.indptr, d.indptr, True, d.sm_scale, rows)
        check(o[idx, h:h + 1].cpu(), lse[idx, h:h + 1].cpu(), ro, rl, torch.bfloat16,
              f"decompress+prefill head {h}")


# ---------------------------------------------------------------------------
# decompression fused into the prefill
# ---------------------------------------------------------------------------

def _latent_to(x: workloads.LatentPrefillInputs, device):
    return workloads.LatentPrefillInputs(
        x.c_kv.to(device), x.k_rope.to(device), x.w_uk.to(device), x.w_uv.to(device),
        x.q.to(device), x.qo_indptr, x.kv_indptr, x.num_heads, x.causal, x.sm_scale)


FUSED_CASES = [
    # (query lengths, key lengths, heads, causal)
    ([1, 31, 32, 33, 127, 128, 129, 257], [1, 31, 32, 33, 127, 128, 129, 257], 3, True),
    ([1, 31, 32, 33, 127, 128, 129, 257], [1, 31, 32, 33, 127, 128, 129, 257], 3, False),
    ([5, 130, 64], [300, 130, 1000], 2, True),       # queries after a prefix
    ([5, 130, 64], [300, 130, 1000], 2, False),
    ([200, 40, 7], [64, 0, 7], 1, True),              # rows that see no key, an empty key range
    ([0, 70, 0, 3], [10, 70, 0, 0], 4, True),         # empty sequences
    ([33, 65, 300], [33, 65, 300], 128, True),        # 128 heads, two parts per head
    ([1000], [1000], 5, True),                        # one sequence, many tiles per workgroup
]


@pytest.mark.parametrize("lens_q,lens_kv,heads,causal", FUSED_CASES)
def test_decompress_prefill_small_parity(lens_q, lens_kv, heads, causal):
    x = workloads.latent_prefill_inputs(lens_q, lens_kv, heads, seed=11, causal=causal)
    g = _latent_to(x, DEV)
    _flush(f"[gpu] fused decompress+prefill q={lens_q} kv={lens_kv} H={heads} causal={causal}")
    o, lse = mra.decompress_prefill(g.q, g.c_kv, g.k_rope, g.w_uk, g.w_uv, x.qo_indptr,
                                    x.kv_indptr, causal, x.sm_scale)
    # the two-call path on the same bytes
    k, v = mra.decompress_kv(g.c_kv, g.k_rope, g.w_uk, g.w_uv, heads)
    o2, lse2 = mra.ragged_prefill(g.q, k, v, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    torch.cuda.synchronize()
    rk, rv = oracle.decompress(x.c_kv, x.k_rope, x.w_uk, x.w_uv, heads)     # fp64
    ro, rl = oracle.prefill(x.q.double(), rk, rv, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    check(o, lse, ro, rl, torch.bfloat16, "fused decompress+prefill")
    # both GPU paths round K/V to bf16 the same way: they agree to within the
    # order of their fp32 sums
    check(o, lse, o2.double().cpu(), lse2.double().cpu(), torch.bfloat16, "fused vs two-call")


@pytest.mark.parametrize("causal", [True, False])
def test_decompress_prefill_running_max_rises_on_every_tile(causal):
    # The forced rescale of the MHA tests through the fused kernel: the keys'
    # RoPE dims come straight from k_rope, so k_rope dim 0 rises with the key
    # index against queries holding 1 in dim 128 (scores climb ~8 per tile).
    lens_q, lens_kv = [300, 129, 64], [300, 129, 700]
    x = workloads.latent_prefill_inputs(lens_q, lens_kv, 2, seed=19, causal=causal)
    q, k_rope = x.q.clone(), x.k_rope.clone()
    q.mul_(0.05)
    q[..., 128] = 1.0
    _rising_keys(k_rope, x.kv_indptr, 0, 0.25)
    x = workloads.LatentPrefillInputs(x.c_kv, k_rope, x.w_uk, x.w_uv, q, x.qo_indptr,
                                      x.kv_indptr, x.num_heads, causal, 1.0)
    g = _latent_to(x, DEV)
    _flush(f"[gpu] fused decompress+prefill, rising scores, causal={causal}")
    o, lse = mra.decompress_prefill(g.q, g.c_kv, g.k_rope, g.w_uk, g.w_uv, x.qo_indptr,
                                    x.kv_indptr, causal, x.sm_scale)
    torch.cuda.synchronize()
    rk, rv = oracle.decompress(x.c_kv, x.k_rope, x.w_uk, x.w_uv, x.num_heads)     # fp64
    ro, rl = oracle.prefill(x.q.double(), rk, rv, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    check(o, lse, ro, rl, torch.bfloat16, "fused decompress+prefill, rising scores")


def test_decompress_prefill_without_lse():
    x = workloads.latent_prefill_inputs([70, 9], [100, 9], 2, seed=12, causal=True)
    g = _latent_to(x, DEV)
    o, lse = mra.decompress_prefill(g.q, g.c_kv, g.k_rope, g.w_uk, g.w_uv, x.qo_indptr,
                                    x.kv_indptr, True, x.sm_scale)
    o_only = mra.decompress_prefill(g.q, g.c_kv, g.k_rope, g.w_uk, g.w_uv, x.qo_indptr,
                                    x.kv_indptr, True, x.sm_scale, return_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o_only)


def test_decompress_prefill_full_size():
    d = workloads.decompress_batch(device=DEV)
    H = d.num_heads
    _flush(f"[gpu] fused decompress+prefill, decompress_batch T={d.indptr[-1]} H={H}")
    o, lse = mra.decompress_prefill(d.q, d.c_kv, d.k_rope, d.w_uk, d.w_uv, d.indptr, d.indptr,
                                    True, d.sm_scale)
    torch.cuda.synchronize()
    _row_properties(o, lse)
    c_kv, k_rope = d.c_kv.cpu(), d.k_rope.cpu()
    rows = sample_rows(d.indptr, block=mra.PREFILL_BLOCK_M, n_random=32, seed=5)
    idx = torch.tensor(rows)
    for h in (0, 3, H - 2, H - 1):
        wk = d.w_uk[:, h * 128:(h + 1) * 128].contiguous().cpu()
        wv = d.w_uv[:, h * 128:(h + 1) * 128].contiguous().cpu()
        rk, rv = oracle.decompress(c_kv, k_rope, wk, wv, 1)           # fp64, all tokens
        qh = head_slice(d.q, h).double()
        ro, rl = oracle.prefill(qh, rk, rv, d.indptr, d.indptr, True, d.sm_scale, rows)
        check(o[idx, h:h + 1].cpu(), lse[idx, h:h + 1].cpu(), ro, rl, torch.bfloat16,
              f"fused decompress+prefill head {h}")
    # every row and head against the two-call path
    k, v = mra.decompress_kv(d.c_kv, d.k_rope, d.w_uk, d.w_uv, H)
    o2, lse2 = mra.ragged_prefill(d.q, k, v, d.indptr, d.indptr, True, d.sm_scale)
    torch.cuda.synchronize()
    del k, v
    err_o = (o.float() - o2.float()).abs().max().item()
    err_l = (lse - lse2).abs().max().item()
    _flush(f"[gpu] fused vs two-call, all rows: O {err_o:.3e}, LSE {err_l:.3e}")
    assert err_o <= TOL[torch.bfloat16][0] and err_l <= TOL[torch.bfloat16][1]
    del d, o, lse, o2, lse2
    torch.cuda.empty_cache()


def _paged_cache_on_gpu(k, v, kv_indptr, page, seed):
    """Page pools [P, page, H, D] holding the contiguous K/V of every sequence
    in a seeded random page order (plus two pages of zeros), built on the GPU,
    and the block table [batch, max_pages]."""
    lens = [b - a for a, b in zip(kv_indptr, kv_indptr[1:])]
    per = [-(-n // page) for n in lens]
    total = sum(per) + 2
    perm = torch.randperm(total, generator=torch.Generator().manual_seed(seed)).tolist()
    h = k.shape[1]
    kc = torch.zeros((total, page, h, k.shape[2]), dtype=k.dtype, device=k.device)
    vc = torch.zeros((total, page, h, v.shape[2]), dtype=v.dtype, device=v.device)
    table = torch.full((len(lens), max(max(per), 1)), -1, dtype=torch.int32)
    i = 0
    for b, n in enumerate(lens):
        for pg in range(per[b]):
            phys = perm[i]
            i += 1
            table[b, pg] = phys
            a = kv_indptr[b] + pg * page
            m = min(page, n - pg * page)
            kc[phys, :m] = k[a:a + m]
            vc[phys, :m] = v[a:a + m]
    return kc, vc, table.to(k.device)


def test_full_size_entry_points_are_bit_identical():
    """The DeepSeek-V3-shaped batch (16 sequences, 128 heads) through the
    device-planned call (eager, then replayed twice from a captured graph
    with eager work and synchronisation between the replays), a plan with
    2-head items, and the paged call (64-key pages in random order): every
    output equals the one-shot call's bit for bit."""
    g = workloads.deepseek_v3_batch(device=DEV)
    t = g.qo_indptr[-1]
    _flush(f"[gpu] full-size entry points: T={t} H={g.num_heads}")
    ref_o, ref_l = mra.ragged_prefill(g.q, g.k, g.v, g.qo_indptr, g.kv_indptr, True, g.sm_scale)
    torch.cuda.synchronize()
    qo_d = torch.tensor(g.qo_indptr, dtype=torch.int32, device=DEV)
    dp = mra.DevicePlan(len(g.qo_indptr) - 1, t, t, g.num_heads)
    o, l = dp.run(g.q, g.k, g.v, qo_d, qo_d, True, g.sm_scale)
    torch.cuda.synchronize()
    assert int(dp.invalid_flag().item()) == 0
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l), "device plan (eager)"
    _flush("[gpu] full-size device plan: graph capture and replays")
    out = torch.zeros_like(ref_o)
    lse = torch.zeros_like(ref_l)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dp.run(g.q, g.k, g.v, qo_d, qo_d, True, g.sm_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    for rep in range(2):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"graph replay {rep}"
        # eager work between the replays
        o2, l2 = mra.ragged_prefill(g.q, g.k, g.v, g.qo_indptr, g.kv_indptr, True, g.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_o) and torch.equal(l2, ref_l), "one-shot between replays"
    del graph, out, lse, o2, l2
    p = mra.Plan(heads_per_item=2).plan(g.qo_indptr, g.kv_indptr, g.num_heads, True).upload()
    o, l = p.run(g.q, g.k, g.v, g.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l), "plan with 2-head items"
    del p, o, l
    _flush("[gpu] full-size paged call (64-key pages)")
    kc, vc, table = _paged_cache_on_gpu(g.k, g.v, g.kv_indptr, 64, seed=70)
    o, l = mra.ragged_prefill_paged(g.q, kc, vc, g.qo_indptr, g.kv_indptr, table, True,
                                    g.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l), "paged"
    del kc, vc, table, o, l, g
    torch.cuda.empty_cache()


def test_plan_run_rejects_tensors_that_do_not_match_the_plan():
    x = _to(workloads.ragged_inputs([40, 90], [50, 90], 4, torch.bfloat16, seed=71), DEV)
    p = mra.Plan().plan(x.qo_indptr, x.kv_indptr, 4, True).upload()
    o, l = p.run(x.q, x.k, x.v, x.sm_scale)
    torch.cuda.synchronize()
    ref_o, ref_l = mra.ragged_prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    for q, k, v in ((x.q[:-1], x.k, x.v),                  # fewer query rows than planned
                    (x.q, x.k[:-1], x.v[:-1]),             # fewer key rows than planned
                    (x.q[:, :2], x.k[:, :2], x.v[:, :2])):  # other head count
        with pytest.raises(mra.MlaError) as e:
            p.run(q.contiguous(), k.contiguous(), v.contiguous(), x.sm_scale)
        assert e.value.status == 5
    torch.cuda.synchronize()


def test_growing_one_shot_does_not_wait_for_other_streams():
    """A one-shot call whose work list outgrows its stream's buffer returns
    while a long kernel on another stream is still running (no device-wide
    synchronisation), and its result is still exact."""
    small = _to(workloads.ragged_inputs([64], [64], 2, torch.bfloat16, seed=72), DEV)
    lens = [700, 300, 1000, 513]
    big = _to(workloads.ragged_inputs(lens, lens, 8, torch.bfloat16, seed=73), DEV)
    ref_o, ref_l = mra.ragged_prefill(big.q, big.k, big.v, big.qo_indptr, big.kv_indptr, True,
                                      big.sm_scale)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(sa):          # this stream's plan starts with a one-item list
        mra.ragged_prefill(small.q, small.k, small.v, small.qo_indptr, small.kv_indptr, True,
                           small.sm_scale)
    torch.cuda.synchronize()
    _flush("[gpu] spin kernel on stream B, growing one-shot call on stream A")
    done_b = torch.cuda.Event()
    with torch.cuda.stream(sb):
        torch.cuda._sleep(2_000_000_000)    # about a second of clock cycles
        done_b.record(sb)
    with torch.cuda.stream(sa):
        o, l = mra.ragged_prefill(big.q, big.k, big.v, big.qo_indptr, big.kv_indptr, True,
                                  big.sm_scale)
    still_running = not done_b.query()
    sa.synchronize()
    torch.cuda.synchronize()
    assert still_running, "the growing call waited for the other stream's kernel"
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


# ---------------------------------------------------------------------------
# weight-absorbed prefill over the latent cache
# ---------------------------------------------------------------------------

def _absorbed_parity(x: workloads.AbsorbedInputs, what, rows=None):
    _flush(f"[gpu] absorbed {what}: Tq={x.qo_indptr[-1]} Tk={x.kv_indptr[-1]} H={x.num_heads} "
           f"causal={x.causal}")
    o, lse = mra.absorbed_prefill(x.q.to(DEV), x.kv.to(DEV), x.qo_indptr, x.kv_indptr, x.causal,
                                  x.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.absorbed(x.q, x.kv, x.qo_indptr, x.kv_indptr, x.causal, x.sm_scale,
                             rows=rows)
    if rows is not None:
        idx = torch.tensor(rows)
        o, lse = o[idx], lse[idx]
    return check(o, lse, ro, rl, torch.bfloat16, f"absorbed {what}")


@pytest.mark.parametrize("case", range(6))
def test_absorbed_random_ragged_batches(case):
    import numpy as np
    rng = np.random.default_rng(3000 + case)
    qo, kv = _random_shape(rng)
    heads = int(rng.choice([1, 4, 16, 32]))
    causal = bool(rng.random() < 0.6)
    x = workloads.absorbed_inputs(qo, kv, heads, seed=4000 + case, causal=causal)
    _absorbed_parity(x, f"random case {case}: qo {qo} kv {kv} H={heads}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("heads", [16, 3, 1])
def test_absorbed_small_parity(causal, heads):
    # ragged lengths spanning several 32-key tiles and 128-row tiles, with tails
    lens = [1, 17, 64, 130, 33]
    x = workloads.absorbed_inputs(lens, lens, heads, seed=11, causal=causal)
    _absorbed_parity(x, f"lens {lens} H={heads}")


@pytest.mark.parametrize("causal", [True, False])
def test_absorbed_context_and_empty_sequences(causal):
    # kv > qo (a context chunk in front), qo > kv (causal rows with no
    # visible key), kv = 0, qo = 0
    qo = [5, 40, 100, 7, 0, 3]
    kv = [37, 40, 300, 0, 9, 1]
    x = workloads.absorbed_inputs(qo, kv, 8, seed=12, causal=causal)
    _absorbed_parity(x, f"qo {qo} kv {kv}")


def test_absorbed_many_heads():
    # 128 heads: one token's rows fill a whole 128-row tile
    lens = [3, 70, 40]
    x = workloads.absorbed_inputs(lens, lens, 128, seed=13, causal=True)
    _absorbed_parity(x, "128 heads")


def test_absorbed_160_heads():
    # 160 rows per token: 128-row tiles start mid-token
    lens = [3, 40, 9]
    x = workloads.absorbed_inputs(lens, [20, 40, 300], 160, seed=66, causal=True)
    _absorbed_parity(x, "160 heads")


def test_absorbed_scale_extremes():
    # large scores (rescale path) and tiny ones
    lens = [200, 90]
    for scale in (1.0, 1e-3):
        x = workloads.absorbed_inputs(lens, lens, 4, seed=14, causal=True, sm_scale=scale)
        _absorbed_parity(x, f"sm_scale {scale}")


@pytest.mark.parametrize("decode", [False, True])
def test_absorbed_running_max_rises_on_every_tile(decode):
    # As for the MHA pass: scores climb by ~8 per 32-key tile, carried by a
    # RoPE dim (512) that the values do not include, so the in-place AGPR
    # rescale of O runs on nearly every tile; the decode shape also splits
    # the keys (each split rescales on its own, then the splits merge).
    if decode:
        lens_q, lens_kv = [1, 1, 1, 1], [2048, 1000, 3000, 64]
    else:
        lens_q, lens_kv = [300, 129, 64], [300, 129, 700]
    x = workloads.absorbed_inputs(lens_q, lens_kv, 4, seed=43, causal=True, sm_scale=1.0)
    q, kv = x.q.clone(), x.kv.clone()
    q.mul_(0.05)
    q[..., 512] = 1.0
    _rising_keys(kv, x.kv_indptr, 512, 0.25)
    x = workloads.AbsorbedInputs(q, kv, x.qo_indptr, x.kv_indptr, x.num_heads, x.causal, x.sm_scale)
    _absorbed_parity(x, f"rising scores decode={decode}")


def test_absorbed_batch_full_size_sampled():
    x = workloads.absorbed_batch(device=DEV)
    _flush(f"[gpu] absorbed_batch Tq={x.qo_indptr[-1]} H={x.num_heads}")
    o, lse = mra.absorbed_prefill(x.q, x.kv, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    torch.cuda.synchronize()
    _row_properties(o, lse)
    rows = sample_rows(x.qo_indptr, block=2048, n_random=24, seed=6)
    ro, rl = oracle.absorbed(x.q.cpu(), x.kv.cpu(), x.qo_indptr, x.kv_indptr, True, x.sm_scale,
                             rows=rows)
    idx = torch.tensor(rows)
    check(o[idx].cpu(), lse[idx].cpu(), ro, rl, torch.bfloat16, "absorbed_batch sampled rows")
    del x, o, lse
    torch.cuda.empty_cache()


def test_absorbed_decode_shape():
    # one new token per sequence over a prefix (a decode step): each sequence
    # is a single tile of H rows that visits every key
    qo = [1, 1, 1, 1]
    kv = [1000, 37, 2500, 1]
    x = workloads.absorbed_inputs(qo, kv, 128, seed=15, causal=True)
    _absorbed_parity(x, "decode shape")


def _latent_paged_cache(x: workloads.AbsorbedInputs, page: int, extra_pages: int, seed: int):
    """Scatter the contiguous latent cache rows of `x` into a page pool in a
    random page order (unused slots and pages hold finite filler) and return
    the pool and the block table (host tensors)."""
    g = torch.Generator().manual_seed(seed)
    lens = [b - a for a, b in zip(x.kv_indptr, x.kv_indptr[1:])]
    per = [-(-n // page) for n in lens]
    total = sum(per) + extra_pages
    perm = torch.randperm(total, generator=g).tolist()
    pool = workloads.randn((total, page, 576), g, torch.bfloat16, "cpu")
    table = torch.full((len(lens), max(max(per), 1)), -1, dtype=torch.int32)
    kv_host = x.kv.cpu()
    i = 0
    for b, n in enumerate(lens):
        for pg in range(per[b]):
            phys = perm[i]
            i += 1
            table[b, pg] = phys
            a = x.kv_indptr[b] + pg * page
            m = min(page, n - pg * page)
            pool[phys, :m] = kv_host[a:a + m]
    return pool, table


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("page", [32, 64, 128])
def test_absorbed_paged_matches_contiguous(causal, page):
    qo_lens = [5, 30, 0, 7, 130, 1]
    kv_lens = [2, 0, 9, 40, 513, 300]
    x = workloads.absorbed_inputs(qo_lens, kv_lens, 16, seed=47, causal=causal)
    _flush(f"[gpu] absorbed paged page={page} causal={causal}")
    pool, table = _latent_paged_cache(x, page, extra_pages=5, seed=page)
    q, kv = x.q.to(DEV), x.kv.to(DEV)
    ref_o, ref_l = mra.absorbed_prefill(q, kv, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    o, l = mra.absorbed_prefill_paged(q, pool.to(DEV), x.qo_indptr, x.kv_indptr, table.to(DEV),
                                      causal, x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_absorbed_paged_prefix_against_the_oracle():
    # new tokens over a paged prefix (causal, bottom-right), checked directly
    # against the oracle on the contiguous bytes
    qo_lens, kv_lens = [64, 1, 9], [200, 96, 257]
    x = workloads.absorbed_inputs(qo_lens, kv_lens, 8, seed=48, causal=True)
    _flush("[gpu] absorbed paged prefix vs oracle")
    pool, table = _latent_paged_cache(x, 64, extra_pages=3, seed=9)
    o, l = mra.absorbed_prefill_paged(x.q.to(DEV), pool.to(DEV), x.qo_indptr, x.kv_indptr,
                                      table.to(DEV), True, x.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.absorbed(x.q, x.kv, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    check(o, l, ro, rl, torch.bfloat16, "absorbed paged prefix")


def test_absorbed_kv_splits_against_the_oracle():
    # few row tiles over long key ranges: the library splits each tile's keys
    # over several items and merges their partial states; rows of one tile
    # see different key counts (causal, 3 tokens x 16 heads in one tile)
    qo, kv = [3, 1, 2], [3000, 777, 64]
    x = workloads.absorbed_inputs(qo, kv, 16, seed=49, causal=True)
    items = mra.absorbed_plan_items(x.qo_indptr, x.kv_indptr, 16, True)
    assert items[:, 8].max() > 0, "expected a KV split"
    _absorbed_parity(x, "KV splits, causal")
    x = workloads.absorbed_inputs(qo, kv, 16, seed=50, causal=False)
    _absorbed_parity(x, "KV splits, non-causal")


def test_absorbed_decode_batch_sampled():
    # a decode step of 16 requests over 4096-token prefixes (8 KV splits)
    x = workloads.absorbed_inputs([1] * 16, [4096] * 16, 128, seed=51, causal=True)
    _flush("[gpu] absorbed decode batch 16 x 4096")
    o, lse = mra.absorbed_prefill(x.q.to(DEV), x.kv.to(DEV), x.qo_indptr, x.kv_indptr, True,
                                  x.sm_scale)
    torch.cuda.synchronize()
    _row_properties(o, lse)
    rows = [0, 5, 11, 15]
    ro, rl = oracle.absorbed(x.q, x.kv, x.qo_indptr, x.kv_indptr, True, x.sm_scale, rows=rows)
    idx = torch.tensor(rows)
    check(o[idx].cpu(), lse[idx].cpu(), ro, rl, torch.bfloat16, "absorbed decode batch")


def test_absorbed_paged_decode_matches_contiguous():
    x = workloads.absorbed_inputs([1, 1, 2], [1500, 300, 2000], 64, seed=52, causal=True)
    pool, table = _latent_paged_cache(x, 64, extra_pages=4, seed=12)
    q, kv = x.q.to(DEV), x.kv.to(DEV)
    ref_o, ref_l = mra.absorbed_prefill(q, kv, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    o, l = mra.absorbed_prefill_paged(q, pool.to(DEV), x.qo_indptr, x.kv_indptr, table.to(DEV),
                                      True, x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


@pytest.mark.parametrize("case", range(6))
def test_absorbed_entry_points_agree_on_random_batches(case):
    # The absorbed routes on one random batch: the one-shot call (checked
    # against the oracle on sampled rows), a plan run twice and a page pool.
    # Odd cases are decode steps (one token per request, 128 heads), where
    # the planner splits the keys and a merge combines the partials.
    import numpy as np
    rng = np.random.default_rng(5000 + case)
    if case % 2:
        batch = int(rng.integers(1, 9))
        qo = [1] * batch
        kv = [int(v) for v in rng.integers(1, 3000, batch)]
        heads, causal = 128, True
    else:
        qo, kv = _random_shape(rng)
        heads = int(rng.choice([2, 8, 16]))
        causal = bool(rng.random() < 0.6)
    page = int(rng.choice([32, 64, 128]))
    x = workloads.absorbed_inputs(qo, kv, heads, seed=6000 + case, causal=causal)
    _flush(f"[gpu] absorbed entry points case {case}: qo {qo} kv {kv} H={heads} "
           f"causal={causal} page={page}")
    q, c = x.q.to(DEV), x.kv.to(DEV)
    ref_o, ref_l = mra.absorbed_prefill(q, c, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    torch.cuda.synchronize()
    n_tok = x.qo_indptr[-1]
    rows = sorted(set(int(r) for r in rng.integers(0, max(n_tok, 1), min(n_tok, 48))))
    if rows:
        ro, rl = oracle.absorbed(x.q, x.kv, x.qo_indptr, x.kv_indptr, causal, x.sm_scale,
                                 rows=rows)
        idx = torch.tensor(rows)
        check(ref_o[idx], ref_l[idx], ro, rl, torch.bfloat16, f"absorbed entry points {case}")
    plan = mra.AbsorbedPlan().plan(x.qo_indptr, x.kv_indptr, heads, causal).upload()
    for layer in range(2):
        o, l = plan.run(q, c, x.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), f"plan, layer {layer}"
    pool, table = _latent_paged_cache(x, page, extra_pages=3, seed=case)
    o, l = mra.absorbed_prefill_paged(q, pool.to(DEV), x.qo_indptr, x.kv_indptr, table.to(DEV),
                                      causal, x.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l), "paged"


def test_absorbed_plan_run_matches_one_shot():
    # plan once, run per layer: bit-identical to the one-shot call, for a
    # prefill batch and for a decode batch with KV splits, contiguous and paged
    for qo, kv, heads, seed in (([5, 130, 33], [5, 130, 300], 16, 60), ([1] * 6, [900] * 6, 128, 61)):
        x = workloads.absorbed_inputs(qo, kv, heads, seed=seed, causal=True)
        q, c = x.q.to(DEV), x.kv.to(DEV)
        plan = mra.AbsorbedPlan().plan(x.qo_indptr, x.kv_indptr, heads, True).upload()
        ref_o, ref_l = mra.absorbed_prefill(q, c, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
        for layer in range(2):
            o, l = plan.run(q, c, x.sm_scale)
            torch.cuda.synchronize()
            assert torch.equal(o, ref_o) and torch.equal(l, ref_l), f"layer {layer}"
        pool, table = _latent_paged_cache(x, 64, extra_pages=2, seed=seed)
        pplan = mra.AbsorbedPlan().plan(x.qo_indptr, x.kv_indptr, heads, True, paged=True).upload()
        o, l = pplan.run_paged(q, pool.to(DEV), table.to(DEV), x.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    # a second layer's inputs through the same plan
    x2 = workloads.absorbed_inputs([1] * 6, [900] * 6, 128, seed=62, causal=True)
    o, l = plan.run(x2.q.to(DEV), x2.kv.to(DEV), x2.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.absorbed(x2.q, x2.kv, x2.qo_indptr, x2.kv_indptr, True, x2.sm_scale)
    check(o, l, ro, rl, torch.bfloat16, "absorbed plan, second layer")


def test_absorbed_one_shot_threads_sharing_a_stream():
    """Decode batches (KV splits, so the per-stream split buffer is shared)
    and a prefill batch from several threads on one stream: every result
    equals the same call made alone."""
    import threading
    shapes = (([1] * 4, [700, 33, 2100, 5]), ([1] * 8, [1500] * 8), ([40, 130], [40, 400]))
    cases = [workloads.absorbed_inputs(qo, kv, 16, seed=70 + i, causal=True)
             for i, (qo, kv) in enumerate(shapes)]
    dev = [(x.q.to(DEV), x.kv.to(DEV)) for x in cases]
    refs = [mra.absorbed_prefill(q, c, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
            for x, (q, c) in zip(cases, dev)]
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    results = [[] for _ in cases]
    errors = []

    def work(i):
        try:
            x, (q, c) = cases[i], dev[i]
            with torch.cuda.stream(stream):
                for _ in range(5):
                    results[i].append(mra.absorbed_prefill(q, c, x.qo_indptr, x.kv_indptr, True,
                                                           x.sm_scale))
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    _flush("[gpu] one-shot absorbed calls from 3 threads on one stream")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (ro, rl), outs in zip(refs, results):
        assert len(outs) == 5
        for o, l in outs:
            assert torch.equal(o, ro) and torch.equal(l, rl)
