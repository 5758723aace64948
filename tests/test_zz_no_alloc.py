"""GPU test of the allocation-free entry point (mla_ragged_prefill_device_plan_noalloc).

Called through the C ABI on two calls in a row, the second with a smaller
input (fewer sequences, heads and tokens, other dtype and causal mode): each
output equals the workspace form's (mla_ragged_prefill_device_plan) bit for
bit and matches the fp64 oracle within the stated tolerances.
"""
import ctypes

import pytest
import torch

import mla_ragged_chunked_amd as mra
import oracle
import workloads
from tests.parity import check

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _noalloc(x, qo_d, kv_d, max_tq, max_tk, out, lse):
    lib = mra.lib()
    return lib.mla_ragged_prefill_device_plan_noalloc(
        x.q.data_ptr(), x.k.data_ptr(), x.v.data_ptr(), qo_d.data_ptr(), kv_d.data_ptr(),
        len(x.qo_indptr) - 1, max_tq, max_tk, x.q.shape[1], int(x.causal), x.sm_scale,
        0 if x.q.dtype == torch.bfloat16 else 1, out.data_ptr(), lse.data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("dummy", [0])
def test_no_alloc_matches_the_workspace_form_on_two_calls(dummy):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    cases = [
        # (qo lens, kv lens, heads, dtype, causal): the second call is smaller
        ([300, 17, 700, 129, 0, 64], [300, 17, 900, 129, 5, 64], 8, torch.bfloat16, True),
        ([5, 64, 33], [40, 64, 1], 2, torch.float32, False),
    ]
    for i, (ql, kl, heads, dtype, causal) in enumerate(cases):
        x = workloads.ragged_inputs(ql, kl, heads, dtype, seed=80 + i, causal=causal)
        g = workloads.PrefillInputs(x.q.to(DEV), x.k.to(DEV), x.v.to(DEV), x.qo_indptr,
                                    x.kv_indptr, heads, causal, x.sm_scale)
        tq, tk = x.qo_indptr[-1], x.kv_indptr[-1]
        print(f"[gpu] no-alloc call {i}: Tq={tq} Tk={tk} H={heads} {dtype} causal={causal}",
              flush=True)
        qo_d = torch.tensor(x.qo_indptr, dtype=torch.int32, device=DEV)
        kv_d = torch.tensor(x.kv_indptr, dtype=torch.int32, device=DEV)
        # the existing entry point, with a workspace
        dp = mra.DevicePlan(len(ql), tq, tk, heads, dtype)
        ref_o, ref_l = dp.run(g.q, g.k, g.v, qo_d, kv_d, causal, x.sm_scale)
        torch.cuda.synchronize()
        assert int(dp.invalid_flag().item()) == 0
        # the allocation-free entry point, outputs pre-filled with garbage
        out = torch.full_like(ref_o, float("nan"))
        lse = torch.full_like(ref_l, float("nan"))
        status = _noalloc(g, qo_d, kv_d, tq, tk, out, lse)
        assert status == 0, mra.lib().mla_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"call {i}: differs"
        ro, rl = oracle.prefill(x.q, x.k, x.v, x.qo_indptr, x.kv_indptr, causal, x.sm_scale)
        check(out, lse, ro, rl, dtype, f"no-alloc call {i}")
