"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than its own formula:
hand-derived golden values, closed forms (one visible key, equal scores),
identities between different calls (split/merge = union, chunked prefill =
one bottom-right causal call, batch = sequences alone), library routines
(torch.tril / softmax / logsumexp / matmul in float64) and bounds.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form.json")
DQK, DVO = 192, 128


def _f(x):
    return float("-inf") if x == "-inf" else float(x)


def _sparse_rows(spec, n, dim):
    t = torch.zeros(n, 1, dim, dtype=torch.float64)
    for r, cols in spec.items():
        for c, val in cols.items():
            t[int(r), 0, int(c)] = float(val)
    return t


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


@pytest.mark.parametrize("case", _golden()["prefill"], ids=lambda c: c["name"])
def test_golden_prefill(case):
    tq, tk = case["qo_indptr"][-1], case["kv_indptr"][-1]
    q = _sparse_rows(case["q"], tq, DQK)
    k = _sparse_rows(case["k"], tk, DQK)
    v = _sparse_rows(case["v"], tk, DVO)
    o, lse = oracle.prefill(q, k, v, case["qo_indptr"], case["kv_indptr"], case["causal"],
                            case["sm_scale"])
    want_o = _sparse_rows(case["expect_o"], tq, DVO)
    want_lse = torch.tensor([_f(x) for x in case["expect_lse"]], dtype=torch.float64)
    assert torch.allclose(o, want_o, atol=1e-12, rtol=0)
    fin = torch.isfinite(want_lse)
    assert torch.equal(torch.isinf(lse[:, 0]), ~fin)
    assert torch.allclose(lse[fin, 0], want_lse[fin], atol=1e-12, rtol=0)


@pytest.mark.parametrize("case", _golden()["merge"], ids=lambda c: c["name"])
def test_golden_merge(case):
    rows, dim = 3, DVO
    o_a = torch.full((rows, dim), _f(case["o_a"]), dtype=torch.float64)
    o_b = torch.full((rows, dim), _f(case["o_b"]), dtype=torch.float64)
    la = torch.full((rows,), _f(case["lse_a"]), dtype=torch.float64)
    lb = torch.full((rows,), _f(case["lse_b"]), dtype=torch.float64)
    o, lse = oracle.merge(o_a, la, o_b, lb)
    assert torch.allclose(o, torch.full_like(o, _f(case["expect_o"])), atol=1e-12, rtol=0)
    want = _f(case["expect_lse"])
    if math.isinf(want):
        assert torch.all(lse == want)
    else:
        assert torch.allclose(lse, torch.full_like(lse, want), atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# Closed forms on random data
# ---------------------------------------------------------------------------

def _rand_case(lens_q, lens_kv, heads, dtype, seed, causal):
    return workloads.ragged_inputs(lens_q, lens_kv, heads, dtype, seed, causal=causal)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_single_visible_key_returns_that_value_row(dtype):
    x = _rand_case([1, 9, 33, 5], [1, 9, 33, 5], 3, dtype, seed=11, causal=True)
    o, lse = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    for b in range(x.batch):
        t, j = x.qo_indptr[b], x.kv_indptr[b]
        for h in range(x.num_heads):
            assert torch.equal(o[t, h], x.v[j, h].double())
            s = x.sm_scale * float(x.q[t, h].double() @ x.k[j, h].double())
            assert abs(float(lse[t, h]) - s) < 1e-12


def test_equal_scores_average_the_visible_values():
    # all keys of a sequence equal -> equal scores -> O = mean of visible V rows
    lens_q, lens_kv = [4, 7, 1], [9, 7, 3]
    x = _rand_case(lens_q, lens_kv, 2, torch.float32, seed=12, causal=True)
    for b in range(x.batch):
        a, e = x.kv_indptr[b], x.kv_indptr[b + 1]
        x.k[a:e] = x.k[a:a + 1]
    o, lse = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    for b in range(x.batch):
        qs, ks = x.qo_indptr[b], x.kv_indptr[b]
        ql, kl = lens_q[b], lens_kv[b]
        for i in range(ql):
            n = min(kl, max(0, kl - ql + i + 1))       # stated visibility count
            for h in range(x.num_heads):
                if n == 0:
                    assert torch.all(o[qs + i, h] == 0) and lse[qs + i, h] == -math.inf
                    continue
                mean = x.v[ks:ks + n, h].double().mean(0)
                assert torch.allclose(o[qs + i, h], mean, atol=1e-12, rtol=0)
                s = x.sm_scale * float(x.q[qs + i, h].double() @ x.k[ks, h].double())
                assert abs(float(lse[qs + i, h]) - (s + math.log(n))) < 1e-12


def _brute(q, k, v, qo, kv, causal, scale):
    """torch float64 softmax / logsumexp with the mask from torch.tril."""
    tq, heads = q.shape[0], q.shape[1]
    o = torch.zeros(tq, heads, v.shape[2], dtype=torch.float64)
    lse = torch.full((tq, heads), -math.inf, dtype=torch.float64)
    for b in range(len(qo) - 1):
        ql, kl = qo[b + 1] - qo[b], kv[b + 1] - kv[b]
        if ql == 0 or kl == 0:
            continue
        for h in range(heads):
            qb = q[qo[b]:qo[b + 1], h].double()
            kb = k[kv[b]:kv[b + 1], h].double()
            vb = v[kv[b]:kv[b + 1], h].double()
            s = (qb @ kb.T) * scale
            if causal:
                keep = torch.tril(torch.ones(ql, kl, dtype=torch.bool), diagonal=kl - ql)
                s = s.masked_fill(~keep, -math.inf)
            rows = torch.isfinite(s).any(1)
            p = torch.softmax(s[rows], dim=1)
            o[qo[b]:qo[b + 1], h][rows] = p @ vb
            lse[qo[b]:qo[b + 1], h][rows] = torch.logsumexp(s[rows], dim=1)
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lens", [([1, 17, 64], [1, 17, 64]), ([5, 0, 12, 3], [9, 4, 12, 1]),
                                  ([8, 2], [3, 30])])
def test_brute_force_library_softmax(causal, lens):
    x = _rand_case(lens[0], lens[1], 4, torch.float32, seed=13, causal=causal)
    o, lse = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    bo, bl = _brute(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
    assert torch.allclose(o, bo, atol=1e-12, rtol=0)
    assert torch.equal(torch.isinf(lse), torch.isinf(bl))
    fin = torch.isfinite(bl)
    assert torch.allclose(lse[fin], bl[fin], atol=1e-12, rtol=0)


def test_per_head_data_is_not_mixed():
    # zero every head but one in Q/K/V: the other heads must come out empty-ish
    x = _rand_case([6], [6], 4, torch.float32, seed=14, causal=True)
    for h in (0, 1, 3):
        x.v[:, h] = 0
    o, _ = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    assert torch.all(o[:, [0, 1, 3]] == 0)
    assert torch.all(o[1:, 2].abs().sum(1) > 0)


def test_split_merge_equals_union():
    g = torch.Generator().manual_seed(15)
    lens_q, lens_kv = [3, 5, 1, 4], [10, 6, 7, 9]
    x = _rand_case(lens_q, lens_kv, 3, torch.float32, seed=15, causal=False)
    full_o, full_l = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, False, x.sm_scale)
    splits = [int(torch.randint(0, n + 1, (1,), generator=g)) for n in lens_kv]
    splits[0] = 0          # an empty left split
    splits[1] = lens_kv[1]  # an empty right split
    ka, va, kb, vb, la, lb = [], [], [], [], [], []
    for b, s in enumerate(splits):
        a, e = x.kv_indptr[b], x.kv_indptr[b + 1]
        ka.append(x.k[a:a + s]); va.append(x.v[a:a + s]); la.append(s)
        kb.append(x.k[a + s:e]); vb.append(x.v[a + s:e]); lb.append(e - a - s)
    ia, ib = workloads.indptr_from_lengths(la), workloads.indptr_from_lengths(lb)
    oa, lsa = oracle.prefill(x.q, torch.cat(ka), torch.cat(va), x.qo_indptr, ia, False, x.sm_scale)
    ob, lsb = oracle.prefill(x.q, torch.cat(kb), torch.cat(vb), x.qo_indptr, ib, False, x.sm_scale)
    mo, ml = oracle.merge(oa, lsa, ob, lsb)
    assert torch.allclose(mo, full_o, atol=1e-12, rtol=0)
    assert torch.allclose(ml, full_l, atol=1e-12, rtol=0)


def test_batch_equals_sequences_alone():
    lens_q, lens_kv = [4, 9, 2], [6, 9, 11]
    x = _rand_case(lens_q, lens_kv, 2, torch.bfloat16, seed=16, causal=True)
    o, lse = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    for b in range(x.batch):
        qs, qe = x.qo_indptr[b], x.qo_indptr[b + 1]
        ks, ke = x.kv_indptr[b], x.kv_indptr[b + 1]
        ob, lb = oracle.prefill(x.q[qs:qe], x.k[ks:ke], x.v[ks:ke], [0, qe - qs], [0, ke - ks],
                                True, x.sm_scale)
        assert torch.equal(ob, o[qs:qe]) and torch.equal(lb, lse[qs:qe])


def test_causal_row_equals_non_causal_prefix():
    n = 12
    x = _rand_case([n], [n], 2, torch.float32, seed=17, causal=True)
    o, lse = oracle.prefill(x.q, x.k, x.v, [0, n], [0, n], True, x.sm_scale)
    for i in range(n):
        oi, li = oracle.prefill(x.q[i:i + 1], x.k[:i + 1], x.v[:i + 1], [0, 1], [0, i + 1],
                                False, x.sm_scale)
        assert torch.allclose(oi[0], o[i], atol=1e-13, rtol=0)
        assert torch.allclose(li[0], lse[i], atol=1e-13, rtol=0)


def test_chunked_prefill_equals_one_bottom_right_causal_call():
    reqs, new, c0, c1, heads = 2, 5, 3, 4, 2
    g = torch.Generator().manual_seed(18)
    r = lambda *s: workloads.randn(s, g, torch.float32, "cpu")
    q = r(reqs * new, heads, DQK)
    k_new, v_new = r(reqs * new, heads, DQK), r(reqs * new, heads, DVO)
    k0, v0 = r(reqs * c0, heads, DQK), r(reqs * c0, heads, DVO)
    k1, v1 = r(reqs * c1, heads, DQK), r(reqs * c1, heads, DVO)
    scale = DQK ** -0.5
    qo = workloads.indptr_from_lengths([new] * reqs)
    i0 = workloads.indptr_from_lengths([c0] * reqs)
    i1 = workloads.indptr_from_lengths([c1] * reqs)
    o, lse, parts = oracle.chunked(q, k_new, v_new, qo, [(k0, v0, i0), (k1, v1, i1)], scale)
    # one call: each request's keys are [ctx0; ctx1; new], causal with kv_len = c0+c1+new
    ks, vs = [], []
    for b in range(reqs):
        ks += [k0[b * c0:(b + 1) * c0], k1[b * c1:(b + 1) * c1], k_new[b * new:(b + 1) * new]]
        vs += [v0[b * c0:(b + 1) * c0], v1[b * c1:(b + 1) * c1], v_new[b * new:(b + 1) * new]]
    kv = workloads.indptr_from_lengths([c0 + c1 + new] * reqs)
    oo, ll = oracle.prefill(q, torch.cat(ks), torch.cat(vs), qo, kv, True, scale)
    assert torch.allclose(o, oo, atol=1e-12, rtol=0)
    assert torch.allclose(lse, ll, atol=1e-12, rtol=0)


def test_output_and_lse_bounds():
    x = _rand_case([20, 3], [25, 3], 3, torch.bfloat16, seed=19, causal=True)
    o, lse = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    for b in range(x.batch):
        ql = x.qo_indptr[b + 1] - x.qo_indptr[b]
        kl = x.kv_indptr[b + 1] - x.kv_indptr[b]
        for i in range(ql):
            t = x.qo_indptr[b] + i
            n = min(kl, max(0, kl - ql + i + 1))
            for h in range(x.num_heads):
                vv = x.v[x.kv_indptr[b]:x.kv_indptr[b] + n, h].double()
                assert torch.all(o[t, h] >= vv.min(0).values - 1e-12)
                assert torch.all(o[t, h] <= vv.max(0).values + 1e-12)
                s = (x.k[x.kv_indptr[b]:x.kv_indptr[b] + n, h].double()
                     @ x.q[t, h].double()) * x.sm_scale
                assert s.max() - 1e-12 <= lse[t, h] <= s.max() + math.log(n) + 1e-12


def test_output_is_linear_in_v():
    x = _rand_case([7, 4], [7, 4], 2, torch.float64, seed=20, causal=True)
    o1, _ = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    o2, _ = oracle.prefill(x.q, x.k, 3.0 * x.v - 1.0, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    assert torch.allclose(o2, 3.0 * o1 - 1.0, atol=1e-12, rtol=0)


def test_sampled_rows_match_full_run():
    x = _rand_case([30, 1, 18], [30, 1, 18], 2, torch.bfloat16, seed=21, causal=True)
    o, lse = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale)
    rows = [48, 0, 29, 30, 31, 5]
    os_, ls = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, True, x.sm_scale, rows)
    assert torch.equal(os_, o[rows]) and torch.equal(ls, lse[rows])


# ---------------------------------------------------------------------------
# merge_state
# ---------------------------------------------------------------------------

def test_merge_is_symmetric_and_associative():
    g = torch.Generator().manual_seed(22)
    st = [(torch.randn(40, 128, generator=g, dtype=torch.float64),
           2 * torch.randn(40, generator=g, dtype=torch.float64)) for _ in range(3)]
    ab = oracle.merge(*st[0], *st[1])
    ba = oracle.merge(*st[1], *st[0])
    assert torch.allclose(ab[0], ba[0], atol=1e-13) and torch.allclose(ab[1], ba[1], atol=1e-13)
    left = oracle.merge(*ab, *st[2])
    bc = oracle.merge(*st[1], *st[2])
    right = oracle.merge(*st[0], *bc)
    assert torch.allclose(left[0], right[0], atol=1e-12) and torch.allclose(left[1], right[1], atol=1e-12)


def test_merge_with_empty_state_is_identity():
    g = torch.Generator().manual_seed(23)
    o = torch.randn(17, 128, generator=g, dtype=torch.float64)
    l = torch.randn(17, generator=g, dtype=torch.float64)
    mo, ml = oracle.merge(o, l, torch.full_like(o, 123.0), torch.full_like(l, -math.inf))
    assert torch.equal(mo, o) and torch.equal(ml, l)


def test_merge_reads_bf16_and_fp32_inputs():
    o_a, l_a, o_b, l_b = workloads.merge_inputs(50, 3, torch.bfloat16, seed=24, neg_inf_frac=0.3)
    mo, ml = oracle.merge(o_a, l_a, o_b, l_b)
    wo, wl = oracle.merge(o_a.double(), l_a.double(), o_b.double(), l_b.double())
    assert torch.equal(mo, wo) and torch.equal(ml, wl)


# ---------------------------------------------------------------------------
# decompression
# ---------------------------------------------------------------------------

def _decomp_small(seed, heads=3, t=5):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s, std=1.0: workloads.randn(s, g, torch.bfloat16, "cpu", std=std)
    return r(t, 512), r(t, 64), r(512, heads * 128, std=512 ** -0.5), r(512, heads * 128, std=512 ** -0.5)


def test_decompress_one_hot_latent_picks_weight_rows():
    c_kv, k_rope, w_uk, w_uv = _decomp_small(25)
    c_kv.zero_()
    c_kv[0, 3] = 1.0
    c_kv[1, 511] = 1.0
    c_kv[2, 7] = 2.0
    c_kv[2, 9] = -1.0
    k, v = oracle.decompress(c_kv, k_rope, w_uk, w_uv, 3)
    wk, wv = w_uk.double().view(512, 3, 128), w_uv.double().view(512, 3, 128)
    assert torch.equal(k[0, :, :128], wk[3]) and torch.equal(v[0], wv[3])
    assert torch.equal(k[1, :, :128], wk[511]) and torch.equal(v[1], wv[511])
    assert torch.equal(k[2, :, :128], 2 * wk[7] - wk[9])
    assert torch.all(k[3:, :, :128] == 0) and torch.all(v[3:] == 0)
    for h in range(3):
        assert torch.equal(k[:, h, 128:], k_rope.double())


def test_decompress_matches_float64_matmul():
    c_kv, k_rope, w_uk, w_uv = _decomp_small(26, heads=2, t=7)
    k, v = oracle.decompress(c_kv, k_rope, w_uk, w_uv, 2)
    mk = (c_kv.double() @ w_uk.double()).view(7, 2, 128)
    mv = (c_kv.double() @ w_uv.double()).view(7, 2, 128)
    assert torch.allclose(k[:, :, :128], mk, atol=1e-12, rtol=0)
    assert torch.allclose(v, mv, atol=1e-12, rtol=0)
    ks, vs = oracle.decompress(c_kv, k_rope, w_uk, w_uv, 2, rows=[6, 2])
    assert torch.equal(ks, k[[6, 2]]) and torch.equal(vs, v[[6, 2]])


# ---------------------------------------------------------------------------
# weight-absorbed MLA over the latent cache (one shared 576-dim row per token)
# ---------------------------------------------------------------------------

def _absorbed_case(lens_q, lens_kv, heads, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    tq, tk = sum(lens_q), sum(lens_kv)
    q = workloads.randn((tq, heads, 576), g, dtype, "cpu")
    kv = workloads.randn((tk, 576), g, dtype, "cpu")
    return q, kv, workloads.indptr_from_lengths(lens_q), workloads.indptr_from_lengths(lens_kv)


def test_absorbed_single_visible_key_returns_that_latent_row():
    q, kv, qo, kvi = _absorbed_case([3, 17, 1], [3, 17, 1], 4, seed=50)
    scale = 192 ** -0.5
    o, lse = oracle.absorbed(q, kv, qo, kvi, True, scale)
    for b in range(3):
        t, j = qo[b], kvi[b]
        for h in range(4):
            assert torch.equal(o[t, h], kv[j, :512].double())
            s = scale * float(q[t, h].double() @ kv[j].double())
            assert abs(float(lse[t, h]) - s) < 1e-12


def test_absorbed_equal_scores_average_the_latent_rows():
    # zero latent part of every query and one shared RoPE part for every key:
    # all visible scores are equal, so O is the mean of the visible latent rows
    lens_q, lens_kv = [5, 9], [7, 9]
    q, kv, qo, kvi = _absorbed_case(lens_q, lens_kv, 3, seed=51)
    q[:, :, :512] = 0
    kv[:, 512:] = kv[0, 512:]
    scale = 0.3
    o, lse = oracle.absorbed(q, kv, qo, kvi, True, scale)
    for b in range(2):
        for i in range(lens_q[b]):
            n = min(lens_kv[b], max(0, lens_kv[b] - lens_q[b] + i + 1))
            t = qo[b] + i
            for h in range(3):
                mean = kv[kvi[b]:kvi[b] + n, :512].double().mean(0)
                assert torch.allclose(o[t, h], mean, atol=1e-12, rtol=0)
                s = scale * float(q[t, h, 512:].double() @ kv[0, 512:].double())
                assert abs(float(lse[t, h]) - (s + math.log(n))) < 1e-12


def _absorbed_brute(q, kv, qo, kvi, causal, scale, dvo=512):
    tq, heads = q.shape[0], q.shape[1]
    o = torch.zeros(tq, heads, dvo, dtype=torch.float64)
    lse = torch.full((tq, heads), -math.inf, dtype=torch.float64)
    for b in range(len(qo) - 1):
        ql, kl = qo[b + 1] - qo[b], kvi[b + 1] - kvi[b]
        if ql == 0 or kl == 0:
            continue
        keys = kv[kvi[b]:kvi[b + 1]].double()
        for h in range(heads):
            s = (q[qo[b]:qo[b + 1], h].double() @ keys.T) * scale
            if causal:
                keep = torch.tril(torch.ones(ql, kl, dtype=torch.bool), diagonal=kl - ql)
                s = s.masked_fill(~keep, -math.inf)
            rows = torch.isfinite(s).any(1)
            o[qo[b]:qo[b + 1], h][rows] = torch.softmax(s[rows], dim=1) @ keys[:, :dvo]
            lse[qo[b]:qo[b + 1], h][rows] = torch.logsumexp(s[rows], dim=1)
    return o, lse


@pytest.mark.parametrize("causal", [True, False])
def test_absorbed_brute_force_library_softmax(causal):
    q, kv, qo, kvi = _absorbed_case([5, 0, 12, 3], [9, 4, 12, 1], 3, seed=52)
    scale = 192 ** -0.5
    o, lse = oracle.absorbed(q, kv, qo, kvi, causal, scale)
    bo, bl = _absorbed_brute(q, kv, qo, kvi, causal, scale)
    assert torch.allclose(o, bo, atol=1e-12, rtol=0)
    assert torch.equal(torch.isinf(lse), torch.isinf(bl))
    fin = torch.isfinite(bl)
    assert torch.allclose(lse[fin], bl[fin], atol=1e-12, rtol=0)


def test_absorbed_equals_mha_over_a_broadcast_cache():
    q, kv, qo, kvi = _absorbed_case([6, 13], [20, 13], 2, seed=53)
    scale = 0.05
    o, lse = oracle.absorbed(q, kv, qo, kvi, True, scale)
    k = kv[:, None, :].expand(-1, 2, -1).contiguous()
    v = kv[:, None, :512].expand(-1, 2, -1).contiguous()
    mo, ml = oracle.prefill(q, k, v, qo, kvi, True, scale)
    assert torch.allclose(o, mo, atol=1e-12, rtol=0) and torch.allclose(lse, ml, atol=1e-12, rtol=0)


def test_weight_absorption_identity_links_the_two_mla_forms():
    # MHA over the decompressed cache (K = [c_kv W_UK_h | k_rope], V = c_kv W_UV_h)
    # equals the absorbed form: queries q_abs = [q_nope W_UK_h^T | q_rope] over
    # the latent rows [c_kv | k_rope], whose 512-dim output is then projected by
    # W_UV_h. Same scores (associativity of the products), so the same LSE.
    heads, lens = 2, [5, 9]
    c_kv, k_rope, w_uk, w_uv = _decomp_small(57, heads=heads, t=sum(lens))
    g = torch.Generator().manual_seed(58)
    q = workloads.randn((sum(lens), heads, DQK), g, torch.float32, "cpu").double()
    ind = workloads.indptr_from_lengths(lens)
    scale = 0.09
    k, v = oracle.decompress(c_kv, k_rope, w_uk, w_uv, heads)
    mo, ml = oracle.prefill(q, k, v, ind, ind, True, scale)
    wk = w_uk.double().view(512, heads, 128)
    wv = w_uv.double().view(512, heads, 128)
    q_abs = torch.cat([torch.einsum("thd,chd->thc", q[:, :, :128], wk), q[:, :, 128:]], dim=-1)
    lat = torch.cat([c_kv.double(), k_rope.double()], dim=-1)
    ao, al = oracle.absorbed(q_abs.contiguous(), lat, ind, ind, True, scale)
    o = torch.einsum("thc,chd->thd", ao, wv)
    assert torch.allclose(al, ml, atol=1e-10, rtol=0)
    assert torch.allclose(o, mo, atol=1e-10, rtol=0)
