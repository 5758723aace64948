"""Helpers for GPU-vs-oracle parity: row sampling and error checks.

Tolerances are the ones stated for this operation: bf16 inputs, max-abs
O error <= 2e-2 and LSE error <= 5e-3; fp32 inputs, 1e-4 and 1e-5. A row
whose oracle LSE is -inf (no visible key) must come back with LSE = -inf
and O exactly 0.
"""
import math
import random

import torch

TOL = {torch.bfloat16: (2e-2, 5e-3), torch.float32: (1e-4, 1e-5)}


def sample_rows(qo_indptr, block=256, n_random=256, seed=0):
    """First/last rows of every sequence, rows on both sides of each tile
    edge, plus seeded random rows."""
    rows = set()
    total = qo_indptr[-1]
    for b in range(len(qo_indptr) - 1):
        qs, qe = qo_indptr[b], qo_indptr[b + 1]
        if qe <= qs:
            continue
        for r in (qs, qs + 1, qe - 2, qe - 1):
            if qs <= r < qe:
                rows.add(r)
        for edge in range(block, qe - qs, block):
            rows.update({qs + edge - 1, qs + edge})
    rng = random.Random(seed)
    for _ in range(min(n_random, total)):
        rows.add(rng.randrange(total))
    return sorted(rows)


def head_slice(t: torch.Tensor, h: int) -> torch.Tensor:
    """[T, 1, D] host copy of head h."""
    return t[:, h:h + 1, :].contiguous().cpu()


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """o_* [n, H, D], lse_* [n, H]; gpu tensors may be on any device."""
    tol_o, tol_l = TOL[dtype]
    o_gpu = o_gpu.detach().double().cpu()
    lse_gpu = lse_gpu.detach().double().cpu()
    empty = torch.isinf(lse_ref)
    assert torch.equal(torch.isneginf(lse_gpu), empty), f"{what}: -inf LSE rows differ"
    if empty.any():
        assert torch.all(o_gpu[empty] == 0), f"{what}: rows with no key must be 0"
    fin = ~empty
    err_o = (o_gpu - o_ref).abs().max().item() if o_ref.numel() else 0.0
    err_l = (lse_gpu[fin] - lse_ref[fin]).abs().max().item() if fin.any() else 0.0
    assert not math.isnan(err_o) and not math.isnan(err_l), f"{what}: NaN"
    assert err_o <= tol_o, f"{what}: O max-abs error {err_o:.3e} > {tol_o}"
    assert err_l <= tol_l, f"{what}: LSE max-abs error {err_l:.3e} > {tol_l}"
    return err_o, err_l
