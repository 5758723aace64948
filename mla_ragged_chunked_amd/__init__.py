"""MLA ragged prefill for MI355X (gfx950): thin Python binding.

Every call marshals torch tensors into pointers and calls the C ABI declared
in include/mla_ragged.h; all arithmetic runs in the HIP kernels of
libmla_ragged.so. PyTorch provides device memory and the current stream
only. There is no fallback: if the library has not been built, or a tensor
is not on a GPU, the call raises.

Functions mirror the C entry points:
  ragged_prefill(q, k, v, qo_indptr, kv_indptr, causal, sm_scale, return_lse=True)
  merge_state(o_a, lse_a, o_b, lse_b, out=None, out_lse=None)
  decompress_kv(c_kv, k_rope, w_uk, w_uv, num_heads)
  absorbed_prefill(q, kv, qo_indptr, kv_indptr, causal, sm_scale, return_lse=True)
  Plan: plan() once per batch, run() once per layer.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = ["ragged_prefill", "ragged_prefill_paged", "ragged_prefill_device_plan_noalloc",
           "merge_state", "decompress_kv", "decompress_prefill",
           "absorbed_prefill", "absorbed_prefill_paged", "absorbed_plan_items", "AbsorbedPlan", "Plan", "DevicePlan", "MlaError", "lib",
           "LIB_PATH", "DQK", "DVO", "DLAT", "DROPE", "PREFILL_BLOCK_M", "EXPORTED_SYMBOLS"]

DQK, DVO, DLAT, DROPE = 192, 128, 512, 64
PREFILL_BLOCK_M = 128          # query rows per work item of the bf16 prefill kernel
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_ragged.so")
_BF16, _FP32 = 0, 1
_DT = {torch.bfloat16: _BF16, torch.float32: _FP32}

EXPORTED_SYMBOLS = [
    "mla_status_string", "mla_last_error", "mla_version", "mla_ragged_prefill",
    "mla_plan_create", "mla_plan_destroy", "mla_ragged_plan", "mla_plan_upload",
    "mla_ragged_run", "mla_plan_info", "mla_plan_items", "mla_plan_items_per_workgroup",
    "mla_plan_set_xcds",
    "mla_plan_set_heads_per_item", "mla_device_plan_workspace_size",
    "mla_ragged_prefill_device_plan", "mla_ragged_prefill_device_plan_noalloc",
    "mla_ragged_prefill_paged",
    "mla_merge_state", "mla_decompress_kv", "mla_decompress_prefill", "mla_absorbed_prefill", "mla_absorbed_plan_items",
    "mla_absorbed_prefill_paged", "mla_absorbed_plan_create", "mla_absorbed_plan_destroy",
    "mla_absorbed_plan_build", "mla_absorbed_plan_upload", "mla_absorbed_run",
    "mla_absorbed_run_paged", "mla_absorbed_plan_info",
]


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        l = lib()
        name = l.mla_status_string(status).decode()
        detail = l.mla_last_error().decode()
        super().__init__(f"{where}: {name}: {detail}")
        self.status = status


_lib = None


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    l = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, C = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                         ctypes.c_char_p)
    sig = {
        "mla_status_string": ([ctypes.c_int], C),
        "mla_last_error": ([], C),
        "mla_version": ([], C),
        "mla_ragged_prefill": ([P, P, P, P, P, I32, I32, I32, F, I32, P, P, P], ctypes.c_int),
        "mla_plan_create": ([ctypes.POINTER(P)], ctypes.c_int),
        "mla_plan_destroy": ([P], None),
        "mla_ragged_plan": ([P, P, P, I32, I32, I32, I32], ctypes.c_int),
        "mla_plan_upload": ([P, P], ctypes.c_int),
        "mla_ragged_run": ([P, P, P, P, I64, I64, I32, F, I32, P, P, P], ctypes.c_int),
        "mla_plan_info": ([P, ctypes.POINTER(I64), ctypes.POINTER(I32), ctypes.POINTER(I32),
                           ctypes.POINTER(I32)], ctypes.c_int),
        "mla_plan_items": ([P, P, I64], ctypes.c_int),
        "mla_plan_items_per_workgroup": ([P, ctypes.POINTER(I32)], ctypes.c_int),
        "mla_plan_set_xcds": ([P, I32], ctypes.c_int),
        "mla_plan_set_heads_per_item": ([P, I32], ctypes.c_int),
        "mla_device_plan_workspace_size": ([I32, I64, I32, I32, ctypes.POINTER(I64)], ctypes.c_int),
        "mla_ragged_prefill_device_plan": ([P, P, P, P, P, I32, I64, I64, I32, I32, F, I32, P, P,
                                            P, I64, P], ctypes.c_int),
        "mla_ragged_prefill_device_plan_noalloc": ([P, P, P, P, P, I32, I64, I64, I32, I32, F,
                                                    I32, P, P, P], ctypes.c_int),
        "mla_ragged_prefill_paged": ([P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, F, I32, P,
                                      P, P], ctypes.c_int),
        "mla_merge_state": ([P, P, P, P, P, P, I64, I32, I32, P], ctypes.c_int),
        "mla_decompress_kv": ([P, P, P, P, I64, I32, P, P, P], ctypes.c_int),
        "mla_decompress_prefill": ([P, P, P, P, P, P, P, I32, I32, I32, F, P, P, P], ctypes.c_int),
        "mla_absorbed_prefill": ([P, P, P, P, I32, I32, I32, F, P, P, P], ctypes.c_int),
        "mla_absorbed_plan_items": ([P, P, I32, I32, I32, P, I64, ctypes.POINTER(I64)],
                                    ctypes.c_int),
        "mla_absorbed_prefill_paged": ([P, P, P, P, P, I32, I32, I32, I32, I32, I32, F, P, P, P],
                                       ctypes.c_int),
        "mla_absorbed_plan_create": ([ctypes.POINTER(P)], ctypes.c_int),
        "mla_absorbed_plan_destroy": ([P], None),
        "mla_absorbed_plan_build": ([P, P, P, I32, I32, I32, I32], ctypes.c_int),
        "mla_absorbed_plan_upload": ([P, P], ctypes.c_int),
        "mla_absorbed_run": ([P, P, P, I64, I64, I32, F, P, P, P], ctypes.c_int),
        "mla_absorbed_run_paged": ([P, P, P, I64, I32, P, I32, I32, I32, F, P, P, P],
                                   ctypes.c_int),
        "mla_absorbed_plan_info": ([P, ctypes.POINTER(I64), ctypes.POINTER(I32)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(l, name)
        fn.argtypes = args
        fn.restype = res
    _lib = l
    return l


def _check(status: int, where: str):
    if status != 0:
        raise MlaError(status, where)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _indptr(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _dev_tensor(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Plan:
    """Work list for one ragged batch: plan once (host), upload, run per layer."""

    def __init__(self, n_xcd: Optional[int] = None, heads_per_item: Optional[int] = None):
        l = lib()
        h = ctypes.c_void_p()
        _check(l.mla_plan_create(ctypes.byref(h)), "mla_plan_create")
        self._h = h
        self._lib = l
        if n_xcd is not None:
            _check(l.mla_plan_set_xcds(h, int(n_xcd)), "mla_plan_set_xcds")
        if heads_per_item is not None:
            _check(l.mla_plan_set_heads_per_item(h, int(heads_per_item)),
                   "mla_plan_set_heads_per_item")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.mla_plan_destroy(h)
            self._h = None

    def plan(self, qo_indptr, kv_indptr, num_heads: int, causal: bool,
             dtype: torch.dtype = torch.bfloat16) -> "Plan":
        qo, kv = _indptr(qo_indptr), _indptr(kv_indptr)
        if len(qo) != len(kv) or len(qo) < 1:
            raise ValueError("qo_indptr and kv_indptr must have the same length >= 1")
        if dtype not in _DT:
            raise ValueError("dtype must be torch.bfloat16 or torch.float32")
        self._qo, self._kv = qo, kv
        _check(self._lib.mla_ragged_plan(self._h, qo.ctypes.data, kv.ctypes.data, len(qo) - 1,
                                         int(num_heads), int(bool(causal)), _DT[dtype]),
               "mla_ragged_plan")
        self.num_heads, self.causal, self.dtype = int(num_heads), bool(causal), dtype
        return self

    def upload(self, device=None) -> "Plan":
        dev = torch.device("cuda") if device is None else torch.device(device)
        with torch.cuda.device(dev):
            _check(self._lib.mla_plan_upload(self._h, _stream(dev)), "mla_plan_upload")
        return self

    def info(self):
        n, bm, nx, nh = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.mla_plan_info(self._h, ctypes.byref(n), ctypes.byref(bm),
                                       ctypes.byref(nx), ctypes.byref(nh)), "mla_plan_info")
        ipw = ctypes.c_int32()
        _check(self._lib.mla_plan_items_per_workgroup(self._h, ctypes.byref(ipw)),
               "mla_plan_items_per_workgroup")
        return {"n_items": n.value, "block_m": bm.value, "n_xcd": nx.value,
                "heads_per_item": nh.value, "items_per_workgroup": ipw.value}

    def items(self) -> np.ndarray:
        n = self.info()["n_items"]
        buf = np.zeros((max(n, 1), 8), dtype=np.int32)
        _check(self._lib.mla_plan_items(self._h, buf.ctypes.data, max(n, 1)), "mla_plan_items")
        return buf[:n]

    def run(self, q, k, v, sm_scale: float, out=None, lse=None, return_lse: bool = True):
        for t, name in ((q, "q"), (k, "k"), (v, "v")):
            _dev_tensor(t, name)
        tq, heads = q.shape[0], q.shape[1]
        if out is None:
            out = torch.empty((tq, heads, DVO), dtype=q.dtype, device=q.device)
        if return_lse and lse is None:
            lse = torch.empty((tq, heads), dtype=torch.float32, device=q.device)
        _dev_tensor(out, "out")
        _check_shapes(q, k, v, out, lse if return_lse else None)
        with torch.cuda.device(q.device):
            # the library checks the sizes against the plan (MLA_ESTATE)
            _check(self._lib.mla_ragged_run(self._h, _ptr(q), _ptr(k), _ptr(v), tq, k.shape[0],
                                            heads, float(sm_scale), _DT[q.dtype], _ptr(out),
                                            _ptr(lse) if return_lse else None,
                                            _stream(q.device)),
                   "mla_ragged_run")
        return (out, lse) if return_lse else out


class DevicePlan:
    """Prefill whose work list is built on the GPU from device indptrs, into a
    workspace this object owns: no host synchronisation and no allocation per
    call, so `run` can be captured in a CUDA/HIP graph and replayed after the
    indptr tensors' contents change (same batch, within max_tq / max_tk)."""

    def __init__(self, batch: int, max_tq: int, max_tk: int, num_heads: int,
                 dtype: torch.dtype = torch.bfloat16, device=None):
        if dtype not in _DT:
            raise ValueError("dtype must be torch.bfloat16 or torch.float32")
        self._lib = lib()
        nbytes = ctypes.c_int64()
        _check(self._lib.mla_device_plan_workspace_size(int(batch), int(max_tq), int(num_heads),
                                                        _DT[dtype], ctypes.byref(nbytes)),
               "mla_device_plan_workspace_size")
        dev = torch.device("cuda") if device is None else torch.device(device)
        self.workspace = torch.zeros(max(nbytes.value, 16), dtype=torch.uint8, device=dev)
        self.batch, self.max_tq, self.max_tk = int(batch), int(max_tq), int(max_tk)
        self.num_heads, self.dtype = int(num_heads), dtype

    def invalid_flag(self) -> torch.Tensor:
        """Device int32 flag: nonzero when some sequence's device indptrs were
        invalid on the last run (those sequences were skipped)."""
        return self.workspace[:4].view(torch.int32)

    def run(self, q, k, v, qo_indptr: torch.Tensor, kv_indptr: torch.Tensor, causal: bool,
            sm_scale: float, out=None, lse=None, return_lse: bool = True):
        for t, name in ((q, "q"), (k, "k"), (v, "v"), (qo_indptr, "qo_indptr"),
                        (kv_indptr, "kv_indptr")):
            _dev_tensor(t, name)
        if qo_indptr.dtype != torch.int32 or kv_indptr.dtype != torch.int32:
            raise ValueError("device indptrs must be int32")
        if qo_indptr.numel() != self.batch + 1 or kv_indptr.numel() != self.batch + 1:
            raise ValueError("device indptrs must have batch + 1 entries")
        if q.shape[0] < self.max_tq or k.shape[0] < self.max_tk:
            raise ValueError("q must hold max_tq rows and k, v max_tk rows")
        if q.shape[1] != self.num_heads or q.dtype != self.dtype:
            raise ValueError("q does not match the plan's heads / dtype")
        if out is None:
            out = torch.empty((q.shape[0], self.num_heads, DVO), dtype=q.dtype, device=q.device)
        if return_lse and lse is None:
            lse = torch.empty((q.shape[0], self.num_heads), dtype=torch.float32, device=q.device)
        _dev_tensor(out, "out")
        _check_shapes(q, k, v, out, lse if return_lse else None)
        with torch.cuda.device(q.device):
            _check(self._lib.mla_ragged_prefill_device_plan(
                _ptr(q), _ptr(k), _ptr(v), _ptr(qo_indptr), _ptr(kv_indptr), self.batch,
                self.max_tq, self.max_tk, self.num_heads, int(bool(causal)), float(sm_scale),
                _DT[q.dtype], _ptr(out), _ptr(lse) if return_lse else None,
                self.workspace.data_ptr(), self.workspace.numel(), _stream(q.device)),
                "mla_ragged_prefill_device_plan")
        return (out, lse) if return_lse else out


NOALLOC_SCRATCH_BYTES = 16 << 20


def ragged_prefill_device_plan_noalloc(q, k, v, qo_indptr: torch.Tensor,
                                       kv_indptr: torch.Tensor, max_tq: int, max_tk: int,
                                       causal: bool, sm_scale: float, out: torch.Tensor,
                                       lse: Optional[torch.Tensor] = None):
    """Device-planned prefill with the library's static scratch as workspace:
    allocates nothing (out, and lse if wanted, are the caller's). Device int32
    indptrs of length batch + 1; q/out hold at least max_tq rows, k/v max_tk.
    Calls that can overlap on one GPU share the scratch and must be ordered."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (qo_indptr, "qo_indptr"),
                    (kv_indptr, "kv_indptr"), (out, "out")):
        _dev_tensor(t, name)
    if qo_indptr.dtype != torch.int32 or kv_indptr.dtype != torch.int32 or \
            qo_indptr.numel() != kv_indptr.numel() or qo_indptr.numel() < 1:
        raise ValueError("device indptrs must be int32 with batch + 1 entries each")
    if q.shape[0] < max_tq or k.shape[0] < max_tk:
        raise ValueError("q must hold max_tq rows and k, v max_tk rows")
    _check_shapes(q, k, v, out, lse)
    with torch.cuda.device(q.device):
        _check(lib().mla_ragged_prefill_device_plan_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(qo_indptr), _ptr(kv_indptr), qo_indptr.numel() - 1,
            int(max_tq), int(max_tk), q.shape[1], int(bool(causal)), float(sm_scale),
            _DT[q.dtype], _ptr(out), _ptr(lse), _stream(q.device)),
            "mla_ragged_prefill_device_plan_noalloc")
    return (out, lse) if lse is not None else out


def _check_shapes(q, k, v, out, lse):
    if q.dtype not in _DT or not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise ValueError("q, k, v, out must share bf16 or fp32")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or out.dim() != 3:
        raise ValueError("q, k, v, out must be [tokens, heads, dim]")
    if q.shape[2] != DQK or k.shape[2] != DQK or v.shape[2] != DVO or out.shape[2] != DVO:
        raise ValueError("head dims must be 192 (q, k) and 128 (v, out)")
    h = q.shape[1]
    if k.shape[1] != h or v.shape[1] != h or out.shape[1] != h:
        raise ValueError("q, k, v, out must have the same number of heads")
    if k.shape[0] != v.shape[0] or out.shape[0] != q.shape[0]:
        raise ValueError("token counts of k/v or q/out differ")
    if lse is not None:
        _dev_tensor(lse, "lse")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (q.shape[0], h):
            raise ValueError("lse must be fp32 [tokens, heads]")


def ragged_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, qo_indptr, kv_indptr,
                   causal: bool, sm_scale: float, return_lse: bool = True,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Ragged MLA prefill. q [Tq,H,192], k [Tk,H,192], v [Tk,H,128] on the GPU;
    host int indptrs of length batch+1. Returns out [Tq,H,128] (and lse [Tq,H]
    fp32, natural log) on the current stream."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _dev_tensor(t, name)
    qo, kv = _indptr(qo_indptr), _indptr(kv_indptr)
    if len(qo) != len(kv) or len(qo) < 1:
        raise ValueError("qo_indptr and kv_indptr must have the same length >= 1")
    if qo[-1] != q.shape[0] or kv[-1] != k.shape[0]:
        raise ValueError("indptr totals do not match the token counts of q / k")
    tq, heads = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((tq, heads, DVO), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((tq, heads), dtype=torch.float32, device=q.device)
    _dev_tensor(out, "out")
    _check_shapes(q, k, v, out, lse if return_lse else None)
    l = lib()
    with torch.cuda.device(q.device):
        _check(l.mla_ragged_prefill(_ptr(q), _ptr(k), _ptr(v), qo.ctypes.data, kv.ctypes.data,
                                    len(qo) - 1, heads, int(bool(causal)), float(sm_scale),
                                    _DT[q.dtype], _ptr(out), _ptr(lse) if return_lse else None,
                                    _stream(q.device)),
               "mla_ragged_prefill")
    return (out, lse) if return_lse else out


def ragged_prefill_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         qo_indptr, kv_indptr, block_table: torch.Tensor, causal: bool,
                         sm_scale: float, return_lse: bool = True,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Ragged MLA prefill over paged K/V. k_cache [P, page, H, 192] and
    v_cache [P, page, H, 128] on the GPU, block_table int32 [batch, max_pages]
    on the GPU, host indptrs (kv_indptr gives the context lengths)."""
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                    (block_table, "block_table")):
        _dev_tensor(t, name)
    qo, kv = _indptr(qo_indptr), _indptr(kv_indptr)
    if len(qo) != len(kv) or len(qo) < 1:
        raise ValueError("qo_indptr and kv_indptr must have the same length >= 1")
    if qo[-1] != q.shape[0]:
        raise ValueError("qo_indptr total does not match the token count of q")
    if k_cache.dim() != 4 or v_cache.dim() != 4 or k_cache.shape[:3] != v_cache.shape[:3]:
        raise ValueError("caches must be [pages, page_size, heads, dim] with matching pages")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
            block_table.shape[0] != len(qo) - 1:
        raise ValueError("block_table must be int32 [batch, max_pages]")
    n_pages, page, heads = k_cache.shape[:3]
    tq = q.shape[0]
    if out is None:
        out = torch.empty((tq, heads, DVO), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((tq, heads), dtype=torch.float32, device=q.device)
    _dev_tensor(out, "out")
    _check_shapes(q, k_cache.view(-1, heads, k_cache.shape[3]),
                  v_cache.view(-1, heads, v_cache.shape[3]), out, lse if return_lse else None)
    with torch.cuda.device(q.device):
        _check(lib().mla_ragged_prefill_paged(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), qo.ctypes.data, kv.ctypes.data,
            _ptr(block_table), block_table.shape[1], page, n_pages, len(qo) - 1, heads,
            int(bool(causal)), float(sm_scale), _DT[q.dtype], _ptr(out),
            _ptr(lse) if return_lse else None, _stream(q.device)),
            "mla_ragged_prefill_paged")
    return (out, lse) if return_lse else out


def merge_state(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
                out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None):
    """Merge two (O, LSE) states over disjoint key sets. o_* [..., 128]
    (bf16 or fp32), lse_* [...] fp32. out/out_lse may alias the inputs."""
    for t, name in ((o_a, "o_a"), (lse_a, "lse_a"), (o_b, "o_b"), (lse_b, "lse_b")):
        _dev_tensor(t, name)
    if o_a.shape != o_b.shape or lse_a.shape != lse_b.shape or o_a.shape[:-1] != lse_a.shape:
        raise ValueError("state shapes differ")
    if o_a.dtype != o_b.dtype or o_a.dtype not in _DT:
        raise ValueError("o_a and o_b must share bf16 or fp32")
    if lse_a.dtype != torch.float32 or lse_b.dtype != torch.float32:
        raise ValueError("lse must be fp32")
    if out is None:
        out = torch.empty_like(o_a)
    if out_lse is None:
        out_lse = torch.empty_like(lse_a)
    _dev_tensor(out, "out")
    _dev_tensor(out_lse, "out_lse")
    if out.shape != o_a.shape or out.dtype != o_a.dtype or out_lse.shape != lse_a.shape:
        raise ValueError("output shapes differ from the inputs")
    rows = lse_a.numel()
    with torch.cuda.device(o_a.device):
        _check(lib().mla_merge_state(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(out),
                                     _ptr(out_lse), rows, o_a.shape[-1], _DT[o_a.dtype],
                                     _stream(o_a.device)),
               "mla_merge_state")
    return out, out_lse


def decompress_kv(c_kv: torch.Tensor, k_rope: torch.Tensor, w_uk: torch.Tensor,
                  w_uv: torch.Tensor, num_heads: int, k_out=None, v_out=None):
    """K [T,H,192] = [c_kv W_UK | k_rope], V [T,H,128] = c_kv W_UV (bf16)."""
    for t, name in ((c_kv, "c_kv"), (k_rope, "k_rope"), (w_uk, "w_uk"), (w_uv, "w_uv")):
        _dev_tensor(t, name)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16")
    t = c_kv.shape[0]
    if c_kv.shape != (t, DLAT) or k_rope.shape != (t, DROPE):
        raise ValueError("c_kv must be [T,512] and k_rope [T,64]")
    if w_uk.shape != (DLAT, num_heads * 128) or w_uv.shape != (DLAT, num_heads * DVO):
        raise ValueError("w_uk / w_uv must be [512, H*128]")
    if k_out is None:
        k_out = torch.empty((t, num_heads, DQK), dtype=torch.bfloat16, device=c_kv.device)
    if v_out is None:
        v_out = torch.empty((t, num_heads, DVO), dtype=torch.bfloat16, device=c_kv.device)
    _dev_tensor(k_out, "k_out")
    _dev_tensor(v_out, "v_out")
    with torch.cuda.device(c_kv.device):
        _check(lib().mla_decompress_kv(_ptr(c_kv), _ptr(k_rope), _ptr(w_uk), _ptr(w_uv), t,
                                       int(num_heads), _ptr(k_out), _ptr(v_out),
                                       _stream(c_kv.device)),
               "mla_decompress_kv")
    return k_out, v_out


def decompress_prefill(q: torch.Tensor, c_kv: torch.Tensor, k_rope: torch.Tensor,
                       w_uk: torch.Tensor, w_uv: torch.Tensor, qo_indptr, kv_indptr,
                       causal: bool, sm_scale: float, return_lse: bool = True,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Ragged MLA prefill with the K/V decompression fused into the kernel:
    q [Tq,H,192], c_kv [Tk,512], k_rope [Tk,64], w_uk / w_uv [512,H*128], all
    bf16 on the GPU; host int indptrs of length batch+1. Equals decompress_kv
    followed by ragged_prefill. Returns out [Tq,H,128] bf16 (and lse [Tq,H]
    fp32, natural log) on the current stream."""
    for t, name in ((q, "q"), (c_kv, "c_kv"), (k_rope, "k_rope"), (w_uk, "w_uk"), (w_uv, "w_uv")):
        _dev_tensor(t, name)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16")
    qo, kv = _indptr(qo_indptr), _indptr(kv_indptr)
    if len(qo) != len(kv) or len(qo) < 1:
        raise ValueError("qo_indptr and kv_indptr must have the same length >= 1")
    if q.dim() != 3 or q.shape[2] != DQK:
        raise ValueError("q must be [tokens, heads, 192]")
    tq, heads = q.shape[0], q.shape[1]
    tk = c_kv.shape[0]
    if c_kv.shape != (tk, DLAT) or k_rope.shape != (tk, DROPE):
        raise ValueError("c_kv must be [Tk,512] and k_rope [Tk,64]")
    if w_uk.shape != (DLAT, heads * DVO) or w_uv.shape != (DLAT, heads * DVO):
        raise ValueError("w_uk / w_uv must be [512, H*128]")
    if qo[-1] != tq or kv[-1] != tk:
        raise ValueError("indptr totals do not match the token counts of q / c_kv")
    if out is None:
        out = torch.empty((tq, heads, DVO), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((tq, heads), dtype=torch.float32, device=q.device)
    _dev_tensor(out, "out")
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (tq, heads, DVO):
        raise ValueError("out must be bf16 [Tq, H, 128]")
    if return_lse:
        _dev_tensor(lse, "lse")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (tq, heads):
            raise ValueError("lse must be fp32 [tokens, heads]")
    with torch.cuda.device(q.device):
        _check(lib().mla_decompress_prefill(_ptr(q), _ptr(c_kv), _ptr(k_rope), _ptr(w_uk),
                                            _ptr(w_uv), qo.ctypes.data, kv.ctypes.data,
                                            len(qo) - 1, heads, int(bool(causal)),
                                            float(sm_scale), _ptr(out),
                                            _ptr(lse) if return_lse else None,
                                            _stream(q.device)),
               "mla_decompress_prefill")
    return (out, lse) if return_lse else out


def absorbed_plan_items(qo_indptr, kv_indptr, num_heads: int, causal: bool) -> np.ndarray:
    """Host work list of the absorbed prefill: int32 [n_items, 12] rows
    {row0, n_rows, seq_row0, kv_hi, kv_start, kv_len, diag_base, kv_lo, part,
    0, 0, 0} (part >= 0: a KV split of its tile)."""
    qo, kv = _indptr(qo_indptr), _indptr(kv_indptr)
    if len(qo) != len(kv) or len(qo) < 1:
        raise ValueError("qo_indptr and kv_indptr must have the same length >= 1")
    l = lib()
    n = ctypes.c_int64(0)
    _check(l.mla_absorbed_plan_items(qo.ctypes.data, kv.ctypes.data, len(qo) - 1, int(num_heads),
                                     int(bool(causal)), None, 0, ctypes.byref(n)),
           "mla_absorbed_plan_items")
    buf = np.zeros((max(n.value, 1), 12), dtype=np.int32)
    _check(l.mla_absorbed_plan_items(qo.ctypes.data, kv.ctypes.data, len(qo) - 1, int(num_heads),
                                     int(bool(causal)), buf.ctypes.data, buf.shape[0],
                                     ctypes.byref(n)),
           "mla_absorbed_plan_items")
    return buf[: n.value]


def absorbed_prefill(q: torch.Tensor, kv: torch.Tensor, qo_indptr, kv_indptr, causal: bool,
                     sm_scale: float, return_lse: bool = True,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Weight-absorbed MLA prefill over the latent cache (bf16): q [Tq,H,576]
    absorbed queries, kv [Tk,576] latent cache rows (c_kv | k_rope) on the
    GPU; host indptrs of length batch+1. Returns out [Tq,H,512] (and lse
    [Tq,H] fp32, natural log) on the current stream."""
    _dev_tensor(q, "q")
    _dev_tensor(kv, "kv")
    if q.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16:
        raise ValueError("q and kv must be bf16")
    dk = DLAT + DROPE
    if q.dim() != 3 or q.shape[2] != dk or kv.dim() != 2 or kv.shape[1] != dk:
        raise ValueError("q must be [Tq,H,576] and kv [Tk,576]")
    qo, kvp = _indptr(qo_indptr), _indptr(kv_indptr)
    if len(qo) != len(kvp) or len(qo) < 1:
        raise ValueError("qo_indptr and kv_indptr must have the same length >= 1")
    if qo[-1] != q.shape[0] or kvp[-1] != kv.shape[0]:
        raise ValueError("indptr totals do not match the token counts of q / kv")
    tq, heads = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((tq, heads, DLAT), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((tq, heads), dtype=torch.float32, device=q.device)
    _dev_tensor(out, "out")
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (tq, heads, DLAT):
        raise ValueError("out must be bf16 [Tq,H,512]")
    if return_lse:
        _dev_tensor(lse, "lse")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (tq, heads):
            raise ValueError("lse must be fp32 [Tq,H]")
    with torch.cuda.device(q.device):
        _check(lib().mla_absorbed_prefill(_ptr(q), _ptr(kv), qo.ctypes.data, kvp.ctypes.data,
                                          len(qo) - 1, heads, int(bool(causal)), float(sm_scale),
                                          _ptr(out), _ptr(lse) if return_lse else None,
                                          _stream(q.device)),
               "mla_absorbed_prefill")
    return (out, lse) if return_lse else out


def absorbed_prefill_paged(q: torch.Tensor, kv_cache: torch.Tensor, qo_indptr, kv_indptr,
                           block_table: torch.Tensor, causal: bool, sm_scale: float,
                           return_lse: bool = True, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None):
    """absorbed_prefill with the latent cache in a page pool kv_cache
    [num_pages, page_size, 576] (bf16) read through block_table [batch,
    max_pages] (int32, on the GPU); host indptrs (only the kv lengths are
    used from kv_indptr)."""
    _dev_tensor(q, "q")
    _dev_tensor(kv_cache, "kv_cache")
    _dev_tensor(block_table, "block_table")
    if q.dtype != torch.bfloat16 or kv_cache.dtype != torch.bfloat16:
        raise ValueError("q and kv_cache must be bf16")
    dk = DLAT + DROPE
    if q.dim() != 3 or q.shape[2] != dk or kv_cache.dim() != 3 or kv_cache.shape[2] != dk:
        raise ValueError("q must be [Tq,H,576] and kv_cache [num_pages,page_size,576]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be int32 [batch, max_pages]")
    qo, kvp = _indptr(qo_indptr), _indptr(kv_indptr)
    if len(qo) != len(kvp) or len(qo) < 1:
        raise ValueError("qo_indptr and kv_indptr must have the same length >= 1")
    if qo[-1] != q.shape[0] or block_table.shape[0] != len(qo) - 1:
        raise ValueError("indptr / block_table do not match q's tokens or the batch")
    tq, heads = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((tq, heads, DLAT), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((tq, heads), dtype=torch.float32, device=q.device)
    _dev_tensor(out, "out")
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (tq, heads, DLAT):
        raise ValueError("out must be bf16 [Tq,H,512]")
    if return_lse:
        _dev_tensor(lse, "lse")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (tq, heads):
            raise ValueError("lse must be fp32 [Tq,H]")
    with torch.cuda.device(q.device):
        _check(lib().mla_absorbed_prefill_paged(
            _ptr(q), _ptr(kv_cache), qo.ctypes.data, kvp.ctypes.data, _ptr(block_table),
            block_table.shape[1], kv_cache.shape[1], kv_cache.shape[0], len(qo) - 1, heads,
            int(bool(causal)), float(sm_scale), _ptr(out), _ptr(lse) if return_lse else None,
            _stream(q.device)),
            "mla_absorbed_prefill_paged")
    return (out, lse) if return_lse else out


class AbsorbedPlan:
    """Work list of the absorbed prefill for one ragged batch: plan once
    (host indptrs), upload, then run per layer (contiguous or paged cache)."""

    def __init__(self):
        self._lib = lib()
        h = ctypes.c_void_p()
        _check(self._lib.mla_absorbed_plan_create(ctypes.byref(h)), "mla_absorbed_plan_create")
        self._h = h
        self.num_heads = 0
        self.tq = 0
        self.batch = 0

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.mla_absorbed_plan_destroy(h)
            self._h = None

    def plan(self, qo_indptr, kv_indptr, num_heads: int, causal: bool,
             paged: bool = False) -> "AbsorbedPlan":
        qo, kv = _indptr(qo_indptr), _indptr(kv_indptr)
        if len(qo) != len(kv) or len(qo) < 1:
            raise ValueError("qo_indptr and kv_indptr must have the same length >= 1")
        _check(self._lib.mla_absorbed_plan_build(self._h, qo.ctypes.data, kv.ctypes.data,
                                                 len(qo) - 1, int(num_heads), int(bool(causal)),
                                                 int(bool(paged))),
               "mla_absorbed_plan_build")
        self.num_heads, self.tq, self.batch = int(num_heads), int(qo[-1]), len(qo) - 1
        return self

    def upload(self, device=None) -> "AbsorbedPlan":
        dev = torch.device("cuda" if device is None else device)
        with torch.cuda.device(dev):
            _check(self._lib.mla_absorbed_plan_upload(self._h, _stream(dev)),
                   "mla_absorbed_plan_upload")
        return self

    def info(self):
        n = ctypes.c_int64(0)
        sp = ctypes.c_int32(0)
        _check(self._lib.mla_absorbed_plan_info(self._h, ctypes.byref(n), ctypes.byref(sp)),
               "mla_absorbed_plan_info")
        return {"n_items": n.value, "kv_splits": sp.value}

    def _outputs(self, q, out, lse, return_lse):
        _dev_tensor(q, "q")
        if q.dtype != torch.bfloat16 or q.dim() != 3 or q.shape[2] != DLAT + DROPE:
            raise ValueError("q must be bf16 [Tq,H,576]")
        if q.shape[0] != self.tq or q.shape[1] != self.num_heads:
            raise ValueError("q does not match the planned tokens / heads")
        if out is None:
            out = torch.empty((self.tq, self.num_heads, DLAT), dtype=torch.bfloat16,
                              device=q.device)
        if return_lse and lse is None:
            lse = torch.empty((self.tq, self.num_heads), dtype=torch.float32, device=q.device)
        _dev_tensor(out, "out")
        if out.dtype != torch.bfloat16 or tuple(out.shape) != (self.tq, self.num_heads, DLAT):
            raise ValueError("out must be bf16 [Tq,H,512]")
        if return_lse:
            _dev_tensor(lse, "lse")
            if lse.dtype != torch.float32 or tuple(lse.shape) != (self.tq, self.num_heads):
                raise ValueError("lse must be fp32 [Tq,H]")
        return out, lse

    def run(self, q, kv, sm_scale: float, out=None, lse=None, return_lse: bool = True):
        _dev_tensor(kv, "kv")
        if kv.dtype != torch.bfloat16 or kv.dim() != 2 or kv.shape[1] != DLAT + DROPE:
            raise ValueError("kv must be bf16 [Tk,576]")
        out, lse = self._outputs(q, out, lse, return_lse)
        with torch.cuda.device(q.device):
            _check(self._lib.mla_absorbed_run(self._h, _ptr(q), _ptr(kv), q.shape[0],
                                              kv.shape[0], q.shape[1], float(sm_scale),
                                              _ptr(out), _ptr(lse) if return_lse else None,
                                              _stream(q.device)),
                   "mla_absorbed_run")
        return (out, lse) if return_lse else out

    def run_paged(self, q, kv_cache, block_table, sm_scale: float, out=None, lse=None,
                  return_lse: bool = True):
        _dev_tensor(kv_cache, "kv_cache")
        _dev_tensor(block_table, "block_table")
        if kv_cache.dtype != torch.bfloat16 or kv_cache.dim() != 3 or \
                kv_cache.shape[2] != DLAT + DROPE:
            raise ValueError("kv_cache must be bf16 [num_pages,page_size,576]")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
                block_table.shape[0] != self.batch:
            raise ValueError("block_table must be int32 [batch, max_pages]")
        out, lse = self._outputs(q, out, lse, return_lse)
        with torch.cuda.device(q.device):
            _check(self._lib.mla_absorbed_run_paged(
                self._h, _ptr(q), _ptr(kv_cache), q.shape[0], q.shape[1], _ptr(block_table),
                block_table.shape[1],
                kv_cache.shape[1], kv_cache.shape[0], float(sm_scale), _ptr(out),
                _ptr(lse) if return_lse else None, _stream(q.device)),
                "mla_absorbed_run_paged")
        return (out, lse) if return_lse else out
