"""fp64 CPU oracle for MLA ragged prefill, merge_state and KV decompression.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product package. It shares no
code with the HIP library; the arithmetic lives in oracle.c (see its header
for the passages each function follows and the readings taken where the
pages are silent).

Parity pins: every function here is pinned by tests that do not reuse its
own formula (single-key rows, equal scores, split/merge identities, a
library-softmax brute force, the chunked-prefill identity, one-hot
decompression and hand-derived golden fixtures).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, FP32, FP64 = 0, 1, 2
_DT = {torch.bfloat16: BF16, torch.float32: FP32, torch.float64: FP64}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    _lib = bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def bind(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_prefill.argtypes = [P, P, P, I, P, P, I, I, I, I, I, D, P, I64, P, P]
    lib.oracle_prefill.restype = I
    lib.oracle_absorbed.argtypes = [P, P, I, P, P, I, I, I, I, I, D, P, I64, P, P]
    lib.oracle_absorbed.restype = I
    lib.oracle_merge.argtypes = [P, P, P, P, I, I, I64, I, P, P]
    lib.oracle_merge.restype = I
    lib.oracle_decompress.argtypes = [P, P, P, P, I, I64, I, I, I, I, I, P, I64, P, P]
    lib.oracle_decompress.restype = I
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    return lib


def _host(t: torch.Tensor) -> torch.Tensor:
    t = t.detach()
    if t.device.type != "cpu":
        t = t.cpu()
    return t.contiguous()


def _i32(a: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def num_threads() -> int:
    return _load().oracle_num_threads()


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, qo_indptr, kv_indptr,
            causal: bool, sm_scale: float, rows: Optional[Sequence[int]] = None):
    """O [n, H, Dvo] and LSE [n, H] in fp64 for the requested query tokens
    (all tokens when rows is None)."""
    lib = _load()
    q, k, v = _host(q), _host(k), _host(v)
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT:
        raise TypeError("q, k, v must share one of bf16 / fp32 / fp64")
    heads, dqk = q.shape[1], q.shape[2]
    dvo = v.shape[2]
    qo = _i32(qo_indptr)
    kv = _i32(kv_indptr)
    batch = len(qo) - 1
    if rows is None:
        n = int(qo[-1])
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = len(rows_arr)
    out = np.zeros((n, heads, dvo), dtype=np.float64)
    lse = np.zeros((n, heads), dtype=np.float64)
    if n == 0 or batch == 0:
        return torch.from_numpy(out), torch.from_numpy(lse)
    rc = lib.oracle_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DT[q.dtype],
                            qo.ctypes.data, kv.ctypes.data, batch, heads, dqk, dvo,
                            int(bool(causal)), float(sm_scale),
                            None if rows_arr is None else rows_arr.ctypes.data, n,
                            out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_prefill failed")
    return torch.from_numpy(out), torch.from_numpy(lse)


def absorbed(q: torch.Tensor, kv: torch.Tensor, qo_indptr, kv_indptr, causal: bool,
             sm_scale: float, dvo: int = 512, rows: Optional[Sequence[int]] = None):
    """Weight-absorbed MLA over the latent cache: q [Tq, H, 576], kv [Tk, 576]
    (one shared row per token, value = its first dvo dims). O [n, H, dvo] and
    LSE [n, H] in fp64."""
    lib = _load()
    q, kv = _host(q), _host(kv)
    if q.dtype != kv.dtype or q.dtype not in _DT:
        raise TypeError("q and kv must share one of bf16 / fp32 / fp64")
    heads, dqk = q.shape[1], q.shape[2]
    if kv.dim() != 2 or kv.shape[1] != dqk:
        raise ValueError("kv must be [Tk, dqk]")
    qo = _i32(qo_indptr)
    kvi = _i32(kv_indptr)
    batch = len(qo) - 1
    if rows is None:
        n = int(qo[-1])
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = len(rows_arr)
    out = np.zeros((n, heads, dvo), dtype=np.float64)
    lse = np.zeros((n, heads), dtype=np.float64)
    if n == 0 or batch == 0:
        return torch.from_numpy(out), torch.from_numpy(lse)
    rc = lib.oracle_absorbed(q.data_ptr(), kv.data_ptr(), _DT[q.dtype], qo.ctypes.data,
                             kvi.ctypes.data, batch, heads, dqk, dvo, int(bool(causal)),
                             float(sm_scale), None if rows_arr is None else rows_arr.ctypes.data,
                             n, out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_absorbed failed")
    return torch.from_numpy(out), torch.from_numpy(lse)


def merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor):
    """Merged (O, LSE) in fp64. o_* [..., D]; lse_* [...] (same leading shape)."""
    lib = _load()
    o_a, o_b, lse_a, lse_b = _host(o_a), _host(o_b), _host(lse_a), _host(lse_b)
    if o_a.dtype != o_b.dtype or lse_a.dtype != lse_b.dtype:
        raise TypeError("both states must share dtypes")
    lead = o_a.shape[:-1]
    dim = o_a.shape[-1]
    rows = int(np.prod(lead)) if len(lead) else 1
    o = np.zeros((rows, dim), dtype=np.float64)
    lse = np.zeros((rows,), dtype=np.float64)
    rc = lib.oracle_merge(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(),
                          _DT[o_a.dtype], _DT[lse_a.dtype], rows, dim,
                          o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_merge failed")
    return (torch.from_numpy(o).reshape(*lead, dim), torch.from_numpy(lse).reshape(lead))


def decompress(c_kv: torch.Tensor, k_rope: torch.Tensor, w_uk: torch.Tensor,
               w_uv: torch.Tensor, num_heads: int, rows: Optional[Sequence[int]] = None):
    """K [n, H, 128+64] and V [n, H, 128] in fp64 for the requested tokens."""
    lib = _load()
    c_kv, k_rope, w_uk, w_uv = _host(c_kv), _host(k_rope), _host(w_uk), _host(w_uv)
    dt = c_kv.dtype
    if not (dt == k_rope.dtype == w_uk.dtype == w_uv.dtype) or dt not in _DT:
        raise TypeError("decompression inputs must share one dtype")
    t, dlat = c_kv.shape
    drope = k_rope.shape[1]
    dnope = w_uk.shape[1] // num_heads
    dvo = w_uv.shape[1] // num_heads
    if rows is None:
        n = t
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = len(rows_arr)
    k_out = np.zeros((n, num_heads, dnope + drope), dtype=np.float64)
    v_out = np.zeros((n, num_heads, dvo), dtype=np.float64)
    if n == 0:
        return torch.from_numpy(k_out), torch.from_numpy(v_out)
    rc = lib.oracle_decompress(c_kv.data_ptr(), k_rope.data_ptr(), w_uk.data_ptr(),
                               w_uv.data_ptr(), _DT[dt], t, num_heads, dlat, dnope, drope,
                               dvo, None if rows_arr is None else rows_arr.ctypes.data, n,
                               k_out.ctypes.data, v_out.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_decompress failed")
    return torch.from_numpy(k_out), torch.from_numpy(v_out)


def chunked(main_q, main_k, main_v, qo_indptr, chunk_kvs, sm_scale, rows=None):
    """Chunked prefill the way the pages run it: the causal pass over the new
    tokens, one non-causal pass per context chunk, then merge_state:
    ((ctx0 (+) ctx1) (+) ...) (+) main.  chunk_kvs: list of (k, v, kv_indptr).
    Returns (final O, final LSE, [partials as (O, LSE)])."""
    parts = []
    for (ck, cv, ckv_indptr) in chunk_kvs:
        parts.append(prefill(main_q, ck, cv, qo_indptr, ckv_indptr, False, sm_scale, rows))
    parts.append(prefill(main_q, main_k, main_v, qo_indptr, qo_indptr, True, sm_scale, rows))
    o, lse = parts[0]
    for (o2, lse2) in parts[1:]:
        o, lse = merge(o, lse, o2, lse2)
    return o, lse, parts
