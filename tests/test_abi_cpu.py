"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects invalid arguments with a status before touching the
device, and its work partitioner covers every (token, head) once."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import mla_ragged_chunked_amd as mra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_ragged.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_what_the_binding_lists():
    assert _declared() == sorted(mra.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", mra.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [s for s in _declared() if s not in exported]
    assert not missing, f"not exported: {missing}"
    lib = mra.lib()
    for s in _declared():
        assert getattr(lib, s) is not None


def test_status_strings_and_version():
    lib = mra.lib()
    assert lib.mla_status_string(0) == b"MLA_OK"
    assert lib.mla_status_string(1) == b"MLA_EINVAL"
    assert lib.mla_status_string(99) == b"MLA_UNKNOWN_STATUS"
    assert lib.mla_version().decode().count(".") == 2


def _prefill(**kw):
    lib = mra.lib()
    qo = np.asarray(kw.pop("qo", [0, 4]), dtype=np.int32)
    kv = np.asarray(kw.pop("kv", [0, 4]), dtype=np.int32)
    args = dict(q=16, k=16, v=16, batch=len(qo) - 1, heads=2, causal=1, scale=0.1, dtype=0,
                out=16, lse=16)
    args.update(kw)
    return lib.mla_ragged_prefill(args["q"], args["k"], args["v"], qo.ctypes.data,
                                  kv.ctypes.data, args["batch"], args["heads"], args["causal"],
                                  args["scale"], args["dtype"], args["out"], args["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 2),
    (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1),
    (dict(scale=-1.0), 1),
    (dict(heads=0), 1),
    (dict(causal=2), 1),
    (dict(batch=-1), 1),
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(k=None), 1),
    (dict(q=24), 1),                       # misaligned
    (dict(lse=8), 1),                      # misaligned lse
    (dict(qo=[1, 4], kv=[0, 4]), 1),       # indptr[0] != 0
    (dict(qo=[0, 4, 2], kv=[0, 4, 5]), 1),  # decreasing
    (dict(qo=[0, 4], kv=[0, 4, 8][:2], heads=70000), 1),
])
def test_prefill_rejects_invalid_arguments(kw, status):
    assert _prefill(**kw) == status
    assert len(mra.lib().mla_last_error()) > 0


def test_empty_batch_is_a_no_op():
    assert _prefill(qo=[0], kv=[0], q=None, k=None, v=None, out=None, lse=None) == 0


def test_merge_and_decompress_reject_invalid_arguments():
    lib = mra.lib()
    assert lib.mla_merge_state(16, 16, 16, 16, 16, 16, 10, 64, 0, None) == 2    # head_dim
    assert lib.mla_merge_state(16, 16, 16, 16, 16, 16, 10, 128, 5, None) == 2   # dtype
    assert lib.mla_merge_state(16, 16, None, 16, 16, 16, 10, 128, 0, None) == 1
    assert lib.mla_merge_state(16, 16, 16, 16, 16, 20, 10, 128, 0, None) == 1   # misaligned
    assert lib.mla_merge_state(16, 16, 16, 16, 16, 16, -1, 128, 0, None) == 1
    assert lib.mla_merge_state(None, None, None, None, None, None, 0, 128, 0, None) == 0
    assert lib.mla_decompress_kv(16, 16, 16, 16, 10, 0, 16, 16, None) == 1
    assert lib.mla_decompress_kv(16, 16, None, 16, 10, 2, 16, 16, None) == 1
    assert lib.mla_decompress_kv(16, 16, 16, 16, -5, 2, 16, 16, None) == 1
    assert lib.mla_decompress_kv(None, None, None, None, 0, 2, None, None, None) == 0


def test_run_before_upload_is_a_state_error():
    p = mra.Plan()
    lib = mra.lib()
    assert lib.mla_ragged_run(p._h, 16, 16, 16, 4, 4, 2, 0.1, 0, 16, 16, None) == 5
    p.plan([0, 4], [0, 4], 2, True)
    assert lib.mla_ragged_run(p._h, 16, 16, 16, 4, 4, 2, 0.1, 0, 16, 16, None) == 5   # not uploaded
    assert b"uploaded" in lib.mla_last_error()


@pytest.mark.parametrize("q_rows,kv_rows,heads,dtype,what", [
    (5, 9, 2, 0, b"q / out rows"),        # q rows differ from qo_indptr[batch]
    (3, 9, 2, 0, b"q / out rows"),
    (4, 8, 2, 0, b"fewer rows"),          # k / v shorter than kv_indptr[batch]
    (4, 9, 3, 0, b"num_heads"),           # other head count
    (4, 9, 2, 1, b"dtype"),               # other dtype
])
def test_run_rejects_tensors_that_do_not_match_the_plan(q_rows, kv_rows, heads, dtype, what):
    # checked before the upload state, so this runs without a GPU
    p = mra.Plan().plan([0, 1, 4], [0, 3, 9], 2, True)
    lib = mra.lib()
    assert lib.mla_ragged_run(p._h, 16, 16, 16, q_rows, kv_rows, heads, 0.1, dtype, 16, 16,
                              None) == 5
    assert what in lib.mla_last_error()
    # sizes that match (k / v may be longer) reach the upload check
    assert lib.mla_ragged_run(p._h, 16, 16, 16, 4, 12, 2, 0.1, 0, 16, 16, None) == 5
    assert b"uploaded" in lib.mla_last_error()


# ---------------------------------------------------------------------------
# work partitioner
# ---------------------------------------------------------------------------

# bf16 plans pair two light tiles while they see at most this many keys,
# and the tiles of a sequence that all see the same keys when there are at
# least PAIR_EQUAL_MIN_TILES of them over at most PAIR_EQUAL_MAX_KEYS keys
PAIR_MAX_KEYS = 512
PAIR_EQUAL_MIN_TILES = 8
PAIR_EQUAL_MAX_KEYS = 4096


def _pairing_pays(qo, kv, bm):
    """Pairing is used only for batches of like sequences: every non-empty
    sequence within 32 query tiles, longest query and key lengths at most
    1.5 times the shortest."""
    ql = [int(qo[b + 1] - qo[b]) for b in range(len(qo) - 1)]
    kl = [int(kv[b + 1] - kv[b]) for b in range(len(qo) - 1)]
    live = [b for b in range(len(ql)) if ql[b] > 0]
    if not live:
        return False
    qs, ks = [ql[b] for b in live], [kl[b] for b in live]
    return -(-max(qs) // bm) <= 32 and 2 * max(qs) <= 3 * min(qs) and 2 * max(ks) <= 3 * min(ks)


def _lim(r, diag0, kv_len):
    return min(kv_len, max(0, diag0 + r + 1))


def _check_plan(qo, kv, heads, causal, dtype_name="bf16", n_xcd=8, heads_per_item=None):
    import torch
    p = mra.Plan(n_xcd=n_xcd, heads_per_item=heads_per_item)
    p.plan(qo, kv, heads, causal, torch.bfloat16 if dtype_name == "bf16" else torch.float32)
    info = p.info()
    items = p.items()
    bm = info["block_m"]
    nh = info["heads_per_item"]
    real = items[items[:, 1] > 0]
    if len(real):
        assert heads % nh == 0
        if heads_per_item:
            assert nh == heads_per_item
    # every (token, head) exactly once
    cover = np.zeros((qo[-1], heads), dtype=np.int64)
    for (q_row0, n_rows, head0, n_heads, kv_start, kv_len, diag0, kv_hi) in real:
        seq = int(np.searchsorted(qo, q_row0, side="right")) - 1
        assert 0 < n_rows <= bm
        assert n_heads == nh and head0 % nh == 0 and 0 <= head0 and head0 + n_heads <= heads
        assert qo[seq] <= q_row0 and q_row0 + n_rows <= qo[seq + 1]     # inside its sequence
        assert (q_row0 - qo[seq]) % bm == 0
        assert kv_start == kv[seq] and kv_len == kv[seq + 1] - kv[seq]
        qo_len = qo[seq + 1] - qo[seq]
        r0 = q_row0 - qo[seq]
        want_diag0 = kv_len - qo_len + r0 if causal else kv_len
        assert diag0 == want_diag0
        assert kv_hi == _lim(n_rows - 1, diag0, kv_len)
        cover[q_row0:q_row0 + n_rows, head0:head0 + n_heads] += 1
    assert np.all(cover == 1)
    # XCD grouping: all tiles of one (sequence, head block) run on one XCD
    # (workgroup w = entry // items_per_workgroup goes to XCD w mod n_xcd)
    ipw = info["items_per_workgroup"]
    # pairs a greedy walk up each sequence's sorted kv_hi values forms: two
    # neighbours while they see at most PAIR_MAX_KEYS keys together
    want_pairs = {}
    for seq in range(len(qo) - 1):
        hs = sorted(int(min(kv[seq + 1] - kv[seq],
                            max(0, (kv[seq + 1] - kv[seq] - (qo[seq + 1] - qo[seq]) + r0 if causal
                                    else kv[seq + 1] - kv[seq]) + min(bm, qo[seq + 1] - qo[seq] - r0))))
                    for r0 in range(0, qo[seq + 1] - qo[seq], bm))
        got, i = [], 0
        if (len(hs) >= PAIR_EQUAL_MIN_TILES and hs[0] > 0 and hs[0] == hs[-1]
                and kv[seq + 1] - kv[seq] <= PAIR_EQUAL_MAX_KEYS):
            # every tile sees the same keys: neighbours pair
            got = [(hs[0], hs[0])] * (len(hs) // 2)
        while not got and i < len(hs):
            if i + 1 < len(hs) and hs[i] + hs[i + 1] <= PAIR_MAX_KEYS:
                got.append((hs[i], hs[i + 1]))
                i += 2
            else:
                i += 1
        want_pairs[seq] = sorted(got)
    pairing = dtype_name == "bf16" and nh == 1 and _pairing_pays(qo, kv, bm)
    if not pairing:
        want_pairs = {seq: [] for seq in want_pairs}
    any_pair = pairing and any(want_pairs.values())
    assert ipw == (2 if any_pair else 1)
    idx = np.nonzero(items[:, 1] > 0)[0]
    groups = {}
    for i in idx:
        groups.setdefault(_group(qo, items[i]), set()).add((i // ipw) % n_xcd)
    assert all(len(v) == 1 for v in groups.values())
    assert len(items) % (n_xcd * ipw) == 0
    if ipw == 2:
        # a workgroup's second entry, when present, follows a real first one
        # of the same (sequence, head), the lighter tile first, and the pairs
        # of every (sequence, head) are the greedy ones
        got = {}
        for w in range(len(items) // 2):
            a, b = items[2 * w], items[2 * w + 1]
            if b[1] == 0:
                continue
            assert a[1] > 0 and _group(qo, a) == _group(qo, b)
            assert a[7] <= b[7] and (a[7] + b[7] <= PAIR_MAX_KEYS or a[7] == b[7])
            got.setdefault(_group(qo, a), []).append((int(a[7]), int(b[7])))
        for seq in range(len(qo) - 1):
            for h in range(heads):
                assert sorted(got.get((seq, h), [])) == want_pairs[seq]
    return items, info


def _group(qo, it):
    return int(np.searchsorted(qo, it[0], side="right")) - 1, int(it[2])


@pytest.mark.parametrize("causal", [True, False])
def test_partition_covers_every_row_once(causal):
    lens = [1, 17, 64, 300, 257, 0, 1000]
    qo = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    _check_plan(qo, qo, 3, causal)
    _check_plan(qo, qo, 8, causal, heads_per_item=4)
    _check_plan(qo, qo, 8, causal, dtype_name="fp32", heads_per_item=8)


def test_partition_handles_ragged_edges():
    # qo > kv (rows with no visible key), kv = 0, qo = 0, kv > qo
    qo_lens = [5, 300, 0, 7, 513]
    kv_lens = [2, 0, 9, 40, 513]
    qo = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32)
    kv = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    items, _ = _check_plan(qo, kv, 2, True)
    # the tiles of the kv = 0 sequence have nothing to visit
    s1 = np.array([it for it in items if it[1] > 0 and _group(qo, it)[0] == 1])
    assert len(s1) and np.all(s1[:, 7] == 0)
    _check_plan(qo, kv, 2, False, dtype_name="fp32")
    _check_plan(qo, kv, 4, True, heads_per_item=2)


def test_partition_defaults_to_one_head_per_item():
    big = np.concatenate([[0], np.cumsum([4096] * 8)]).astype(np.int32)
    _, info = _check_plan(big, big, 128, True)
    assert info["heads_per_item"] == 1
    _, info = _check_plan(big, big, 128, True, heads_per_item=8)
    assert info["heads_per_item"] == 8


def test_partition_rejects_a_head_block_that_does_not_divide():
    import torch
    p = mra.Plan(heads_per_item=3)
    with pytest.raises(RuntimeError):
        p.plan([0, 64], [0, 64], 4, True, torch.bfloat16)
    lib = mra.lib()
    assert lib.mla_plan_set_heads_per_item(p._h, -1) == 1


def test_partition_balances_xcds_and_orders_heaviest_first():
    lens = [16, 32768, 40, 5000, 2000, 100, 8191, 3]
    qo = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    for hpi in (None, 4):
        items, info = _check_plan(qo, qo, 16, True, heads_per_item=hpi)
        ipw = info["items_per_workgroup"]
        xcd_of = (np.arange(len(items)) // ipw) % 8
        cost = np.where(items[:, 1] > 0, (items[:, 7] + 64) * items[:, 3], 0).astype(np.int64)
        per_xcd = [cost[xcd_of == x].sum() for x in range(8)]
        group_cost = {}
        for it, c in zip(items, cost):
            if it[1] > 0:
                key = _group(qo, it)
                group_cost[key] = group_cost.get(key, 0) + c
        assert max(per_xcd) - min(per_xcd) <= max(group_cost.values())
        # inside one XCD queue the groups come heaviest first
        for x in range(8):
            seen = []
            for it in items[xcd_of == x]:
                if it[1] > 0 and (not seen or seen[-1] != _group(qo, it)):
                    seen.append(_group(qo, it))
            costs = [group_cost[k] for k in seen]
            assert costs == sorted(costs, reverse=True)


def test_partition_without_xcd_grouping_has_no_padding():
    lens = [100, 700, 3]
    qo = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    items, info = _check_plan(qo, qo, 4, True, n_xcd=1)
    # every workgroup has work (only a single tile's partner entry is empty)
    ipw = info["items_per_workgroup"]
    assert np.all(items[::ipw, 1] > 0) and info["n_xcd"] == 1


# ---------------------------------------------------------------------------
# device-planned prefill: host-side checks (no HIP call is made)
# ---------------------------------------------------------------------------

def _ws_size(batch, max_tq, heads, dtype=0):
    import ctypes
    n = ctypes.c_int64(-1)
    st = mra.lib().mla_device_plan_workspace_size(batch, max_tq, heads, dtype, ctypes.byref(n))
    return st, n.value


def test_device_plan_workspace_size():
    st, a = _ws_size(16, 25729, 128)
    assert st == 0 and a > 0
    # the work list bound: 8 XCD bins x ceil(H/8) heads x (tiles of max_tq + one per sequence)
    bm = 128
    assert a >= 8 * 16 * (-(-25729 // bm) + 16) * 32
    assert _ws_size(32, 25729, 128)[1] > a and _ws_size(16, 60000, 128)[1] > a
    assert _ws_size(0, 0, 1)[0] == 0
    assert _ws_size(4097, 100, 4)[0] == 1          # batch beyond the device sort
    assert _ws_size(4, 100, 0)[0] == 1
    assert _ws_size(4, 100, 4, dtype=7)[0] == 2


def test_device_plan_rejects_invalid_arguments_before_any_hip_call():
    l = mra.lib()
    st, need = _ws_size(2, 64, 4)
    args = [16, 16, 16, 16, 16, 2, 64, 64, 4, 1, 0.1, 0, 16, 16, 16, need, None]

    def call(**kw):
        a = list(args)
        names = ["q", "k", "v", "qo", "kv", "batch", "max_tq", "max_tk", "heads", "causal",
                 "scale", "dtype", "out", "lse", "ws", "ws_bytes", "stream"]
        for key, val in kw.items():
            a[names.index(key)] = val
        return l.mla_ragged_prefill_device_plan(*a)

    assert call(ws_bytes=need - 1) == 1                # workspace too small
    assert call(ws=None) == 1
    assert call(ws=8) == 1                             # misaligned workspace
    assert call(scale=float("nan")) == 1
    assert call(causal=2) == 1
    assert call(batch=4097) == 1
    assert call(qo=None) == 1
    assert call(dtype=5) == 2
    assert call(max_tq=-1) == 1
    assert call(max_tq=(1 << 31) // 4 + 1) == 2        # tokens x heads beyond 2^31
    assert call(batch=0) == 0                          # no-op


def test_paged_prefill_rejects_invalid_arguments_before_any_hip_call():
    import numpy as np
    l = mra.lib()
    qo = np.array([0, 40, 100], dtype=np.int32)
    kv = np.array([0, 64, 192], dtype=np.int32)      # contexts of 64 and 128 keys
    base = dict(q=16, k=16, v=16, qo=qo.ctypes.data, kv=kv.ctypes.data, table=16, max_pages=2,
                page=64, pages=8, batch=2, heads=4, causal=1, scale=0.1, dtype=0, out=16, lse=16,
                stream=None)
    order = ["q", "k", "v", "qo", "kv", "table", "max_pages", "page", "pages", "batch", "heads",
             "causal", "scale", "dtype", "out", "lse", "stream"]

    def call(**kw):
        a = dict(base, **kw)
        return l.mla_ragged_prefill_paged(*[a[n] for n in order])

    assert call(page=48) == 1                     # not a multiple of 32
    assert call(page=0) == 1
    assert call(max_pages=1) == 1                 # 128 keys do not fit 1 page of 64
    assert call(table=None) == 1
    assert call(table=18) == 1                    # misaligned table
    assert call(pages=0) == 1
    assert call(scale=-1.0) == 1
    assert call(dtype=3) == 2


# ---------------------------------------------------------------------------
# weight-absorbed prefill: work list and argument checks (no HIP call)
# ---------------------------------------------------------------------------

ABS_BM = 128


def _check_latent_plan(qo_lens, kv_lens, heads, causal):
    qo = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32)
    kv = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    items = mra.absorbed_plan_items(qo, kv, heads, causal)
    assert len(items) % 8 == 0
    real = items[items[:, 1] > 0]
    assert not np.any(items[items[:, 1] == 0]), "padding items are all zero"
    parts = set(int(p) for p in real[:, 8])
    splits = 1 if parts <= {-1} else len(parts)
    assert parts == ({-1} if splits == 1 else set(range(splits)))
    cover = np.zeros(int(qo[-1]) * heads, dtype=np.int64)
    ranges = {}
    groups = {}
    for i, (row0, n_rows, seq_row0, kv_hi, kv_start, kv_len, diag_base, kv_lo, part,
            p0, p1, p2) in enumerate(items):
        if n_rows == 0:
            continue
        assert 0 < n_rows <= ABS_BM and p0 == p1 == p2 == 0
        seq = int(np.searchsorted(qo * heads, row0, side="right")) - 1
        assert seq_row0 == qo[seq] * heads
        assert (row0 - seq_row0) % ABS_BM == 0
        assert row0 + n_rows <= qo[seq + 1] * heads        # inside its sequence
        assert kv_start == kv[seq] and kv_len == kv[seq + 1] - kv[seq]
        qo_len = qo[seq + 1] - qo[seq]
        assert diag_base == (kv_len - qo_len if causal else kv_len)
        assert kv_lo % 32 == 0 and 0 <= kv_lo <= kv_hi
        cover[row0:row0 + n_rows] += 1
        ranges.setdefault(row0, []).append((int(part), int(kv_lo), int(kv_hi)))
        groups.setdefault(seq, set()).add(i % 8)
    assert np.all(cover == splits)
    # the splits of a tile cover the keys its last row sees, in order, once
    for row0, rs in ranges.items():
        seq = int(np.searchsorted(qo * heads, row0, side="right")) - 1
        n_rows = next(int(it[1]) for it in real if it[0] == row0)
        qo_len, kv_len = qo[seq + 1] - qo[seq], kv[seq + 1] - kv[seq]
        diag = kv_len - qo_len if causal else kv_len
        last_tok = (row0 + n_rows - 1 - qo[seq] * heads) // heads
        want_hi = min(kv_len, max(0, diag + last_tok + 1))
        rs.sort()
        assert [r[0] for r in rs] == ([-1] if splits == 1 else list(range(splits)))
        assert rs[0][1] == 0 and rs[-1][2] == want_hi
        for (pa, lo_a, hi_a), (pb, lo_b, hi_b) in zip(rs, rs[1:]):
            assert hi_a == lo_b or (hi_a == want_hi and lo_b >= want_hi - 31)
    return items, groups, splits


@pytest.mark.parametrize("causal", [True, False])
def test_absorbed_partition_covers_every_row_once(causal):
    _check_latent_plan([1, 17, 64, 300, 0, 129], [1, 17, 64, 300, 5, 129], 16, causal)
    _check_latent_plan([5, 300, 0, 7, 513], [2, 0, 9, 40, 513], 3, causal)   # odd H
    _check_latent_plan([1, 2, 3], [1, 2, 3], 1, causal)


def test_absorbed_partition_keeps_short_sequences_on_one_xcd():
    # at most 256 tiles per group: a sequence with fewer tiles stays on one XCD
    items, groups, splits = _check_latent_plan([100, 40, 4000, 8], [100, 40, 4000, 8], 16, True)
    assert splits == 1
    assert len(groups[0]) == 1 and len(groups[1]) == 1 and len(groups[3]) == 1
    assert len(groups[2]) == 2         # 4000 x 16 rows = 500 tiles: two groups


def test_absorbed_partition_splits_keys_when_tiles_are_few():
    # a decode step (one token per sequence) over long prefixes: the keys of
    # each tile are shared out over several items
    _, _, splits = _check_latent_plan([1] * 16, [4096] * 16, 128, True)
    assert splits == 16              # 16 tiles -> 256 items, one per CU
    _, _, splits = _check_latent_plan([1] * 64, [4096] * 64, 128, True)
    assert splits == 4
    _, _, splits = _check_latent_plan([1] * 4, [200, 37, 300, 1], 128, True)
    assert 1 < splits <= 2           # at least four 32-key tiles per split
    _, _, splits = _check_latent_plan([1] * 4, [64, 37, 100, 1], 128, False)
    assert splits == 1               # too few keys to split
    _, _, splits = _check_latent_plan([2048] * 2, [2048] * 2, 128, True)
    assert splits == 1               # enough row tiles


def test_absorbed_prefill_rejects_invalid_arguments_before_any_hip_call():
    lib = mra.lib()
    qo = np.array([0, 4], dtype=np.int32)
    kv = np.array([0, 4], dtype=np.int32)
    bad_qo = np.array([0, 4, 2], dtype=np.int32)
    args = lambda **kw: dict(dict(q=16, kv=16, qo=qo.ctypes.data, kvp=kv.ctypes.data, batch=1,
                                  heads=2, causal=1, scale=0.1, out=16, lse=16), **kw)
    def call(**kw):
        a = args(**kw)
        return lib.mla_absorbed_prefill(a["q"], a["kv"], a["qo"], a["kvp"], a["batch"],
                                        a["heads"], a["causal"], a["scale"], a["out"], a["lse"],
                                        None)
    assert call(scale=0.0) == 1
    assert call(scale=float("nan")) == 1
    assert call(heads=0) == 1
    assert call(causal=2) == 1
    assert call(batch=-1) == 1
    assert call(q=None) == 1
    assert call(kv=None) == 1
    assert call(out=20) == 1                          # misaligned
    assert call(qo=bad_qo.ctypes.data, kvp=np.array([0, 1, 2], dtype=np.int32).ctypes.data,
                batch=2) == 1                         # decreasing indptr
    assert call(qo=np.array([1, 4], dtype=np.int32).ctypes.data) == 1   # indptr[0] != 0
    big = np.array([0, 1 << 24], dtype=np.int32)
    assert call(qo=big.ctypes.data, heads=256) == 1  # tokens x heads >= 2^31
    # nothing to do: returns before any HIP call
    empty = np.array([0], dtype=np.int32)
    assert call(qo=empty.ctypes.data, kvp=empty.ctypes.data, batch=0, q=None, kv=None,
                out=None, lse=None) == 0


def test_absorbed_paged_rejects_invalid_arguments_before_any_hip_call():
    lib = mra.lib()
    qo = np.array([0, 4], dtype=np.int32)
    kv = np.array([0, 64], dtype=np.int32)
    bt = np.zeros(4, dtype=np.int32)

    def call(page_size=32, max_pages=2, num_pages=4, table=bt.ctypes.data, kvp=kv):
        return lib.mla_absorbed_prefill_paged(16, 16, qo.ctypes.data, kvp.ctypes.data, table,
                                              max_pages, page_size, num_pages, 1, 2, 1, 0.1,
                                              16, 16, None)
    assert call(page_size=48) == 1                    # not a multiple of 32
    assert call(page_size=0) == 1
    assert call(max_pages=0) == 1
    assert call(num_pages=0) == 1
    assert call(table=None) == 1
    assert call(table=bt.ctypes.data + 2) == 1        # misaligned table
    assert call(kvp=np.array([0, 65], dtype=np.int32)) == 1   # context > max_pages x page_size


def test_absorbed_plan_states_and_info_without_a_gpu():
    import ctypes
    lib = mra.lib()
    p = mra.AbsorbedPlan()
    # not built: every run is a state error, before any HIP call
    assert lib.mla_absorbed_run(p._h, 16, 16, 2, 8192, 128, 0.1, 16, 16, None) == 5
    assert lib.mla_absorbed_plan_info(p._h, None, None) == 5
    qo = np.array([0, 1, 2], dtype=np.int32)
    kv = np.array([0, 4096, 8192], dtype=np.int32)
    p.plan(qo, kv, 128, True)
    info = p.info()
    assert info["kv_splits"] > 1 and info["n_items"] % 8 == 0
    # built, not uploaded
    assert lib.mla_absorbed_run(p._h, 16, 16, 2, 8192, 128, 0.1, 16, 16, None) == 5
    assert b"uploaded" in lib.mla_last_error()
    # tensors that do not match the plan: state errors, before the upload check
    for q_rows, kv_rows, heads, what in ((3, 8192, 128, b"q / out rows"),
                                         (2, 8191, 128, b"fewer rows"),
                                         (2, 8192, 64, b"num_heads")):
        assert lib.mla_absorbed_run(p._h, 16, 16, q_rows, kv_rows, heads, 0.1, 16, 16,
                                    None) == 5
        assert what in lib.mla_last_error()
    # built for a contiguous cache: a paged run is a state error
    bt = np.zeros(4, dtype=np.int32)
    assert lib.mla_absorbed_run_paged(p._h, 16, 16, 2, 128, bt.ctypes.data, 128, 32, 256, 0.1,
                                      16, 16, None) == 5
    assert lib.mla_absorbed_run_paged(p._h, 16, 16, 2, 128, bt.ctypes.data, 128, 48, 256, 0.1,
                                      16, 16, None) == 1          # page size
    with pytest.raises(RuntimeError):
        p.plan([0, 3, 2], [0, 1, 2], 4, True)              # decreasing indptr
    assert lib.mla_absorbed_plan_build(p._h, qo.ctypes.data, kv.ctypes.data, 2, 4, 1, 2) == 1


def test_binding_refuses_host_tensors():
    """No CPU fallback: every compute entry of the binding rejects tensors that
    are not on the GPU before it reaches the library."""
    import torch
    t, h = 5, 2
    q = torch.zeros((t, h, 192), dtype=torch.bfloat16)
    k = torch.zeros((t, h, 192), dtype=torch.bfloat16)
    v = torch.zeros((t, h, 128), dtype=torch.bfloat16)
    ind = [0, t]
    with pytest.raises(ValueError, match="GPU tensor"):
        mra.ragged_prefill(q, k, v, ind, ind, True, 0.1)
    o = torch.zeros((t, h, 128), dtype=torch.bfloat16)
    l = torch.zeros((t, h), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        mra.merge_state(o, l, o, l)
    with pytest.raises(ValueError, match="GPU tensor"):
        mra.decompress_kv(torch.zeros((t, 512), dtype=torch.bfloat16),
                          torch.zeros((t, 64), dtype=torch.bfloat16),
                          torch.zeros((512, h * 128), dtype=torch.bfloat16),
                          torch.zeros((512, h * 128), dtype=torch.bfloat16), h)
    with pytest.raises(ValueError, match="GPU tensor"):
        mra.absorbed_prefill(torch.zeros((t, h, 576), dtype=torch.bfloat16),
                             torch.zeros((t, 576), dtype=torch.bfloat16), ind, ind, True, 0.1)
    with pytest.raises(ValueError, match="GPU tensor"):
        mra.decompress_prefill(q, torch.zeros((t, 512), dtype=torch.bfloat16),
                               torch.zeros((t, 64), dtype=torch.bfloat16),
                               torch.zeros((512, h * 128), dtype=torch.bfloat16),
                               torch.zeros((512, h * 128), dtype=torch.bfloat16), ind, ind,
                               True, 0.1)


def test_binding_block_m_matches_the_planner():
    # the full-size GPU tests sample rows on both sides of every query-tile
    # edge using the binding's constant
    p = mra.Plan().plan([0, 300], [0, 300], 2, True)
    assert p.info()["block_m"] == mra.PREFILL_BLOCK_M


def test_noalloc_prefill_rejects_bad_calls_before_any_hip_call():
    lib = mra.lib()
    qo = np.array([0, 10], dtype=np.int32)
    f = lib.mla_ragged_prefill_device_plan_noalloc
    # a batch whose device-plan workspace exceeds the 16 MiB scratch array
    # (128 heads, 10^6 query tokens: ~32 MB of work list): unsupported
    assert f(16, 16, 16, qo.ctypes.data, qo.ctypes.data, 1, 1_000_000, 1_000_000, 128, 1,
             0.1, 0, 16, 16, None) == 2
    assert b"scratch" in lib.mla_last_error()
    # the same checks as the workspace form
    assert f(16, 16, 16, qo.ctypes.data, qo.ctypes.data, 1, 10, 10, 0, 1, 0.1, 0, 16, 16,
             None) == 1                                        # num_heads
    assert f(16, 16, 16, qo.ctypes.data, qo.ctypes.data, 5000, 10, 10, 4, 1, 0.1, 0, 16, 16,
             None) == 1                                        # batch > 4096
    assert f(16, 16, 16, qo.ctypes.data, qo.ctypes.data, 1, 10, 10, 4, 1, float("nan"), 0, 16,
             16, None) == 1                                    # sm_scale
    assert f(16, 16, 16, None, None, 1, 10, 10, 4, 1, 0.1, 0, 16, 16, None) == 1
    assert f(None, None, None, None, None, 0, 0, 0, 4, 1, 0.1, 0, None, None, None) == 0
    # the largest skewed workload fits: 128 heads, 262,144 tokens, 64 sequences
    n = ctypes.c_int64()
    assert lib.mla_device_plan_workspace_size(64, 262144, 128, 0, ctypes.byref(n)) == 0
    assert n.value <= mra.NOALLOC_SCRATCH_BYTES


def test_decompress_prefill_rejects_invalid_arguments_before_any_hip_call():
    lib = mra.lib()
    qo = np.array([0, 4], dtype=np.int32)
    kv = np.array([0, 4], dtype=np.int32)
    def call(**kw):
        a = dict(q=16, c=16, r=16, wk=16, wv=16, qo=qo.ctypes.data, kvp=kv.ctypes.data, batch=1,
                 heads=2, causal=1, scale=0.1, out=16, lse=16)
        a.update(kw)
        return lib.mla_decompress_prefill(a["q"], a["c"], a["r"], a["wk"], a["wv"], a["qo"],
                                          a["kvp"], a["batch"], a["heads"], a["causal"],
                                          a["scale"], a["out"], a["lse"], None)
    assert call(scale=0.0) == 1
    assert call(scale=float("inf")) == 1
    assert call(heads=0) == 1
    assert call(heads=70000) == 1
    assert call(causal=-1) == 1
    assert call(batch=-1) == 1
    assert call(qo=None) == 1
    for name in ("q", "c", "r", "wk", "wv", "out"):
        assert call(**{name: None}) == 1, name
    for name in ("q", "c", "r", "wk", "wv", "out", "lse"):
        assert call(**{name: 24}) == 1, name              # misaligned
    assert call(qo=np.array([0, 4, 2], dtype=np.int32).ctypes.data,
                kvp=np.array([0, 1, 2], dtype=np.int32).ctypes.data, batch=2) == 1
    assert call(kvp=np.array([2, 4], dtype=np.int32).ctypes.data) == 1   # indptr[0] != 0
    big = np.array([0, 1 << 24], dtype=np.int32)
    assert call(qo=big.ctypes.data, heads=256) == 2       # tokens x heads >= 2^31
    # nothing to do: returns before any HIP call
    empty = np.array([0], dtype=np.int32)
    assert call(qo=empty.ctypes.data, kvp=empty.ctypes.data, batch=0, q=None, c=None, r=None,
                wk=None, wv=None, out=None, lse=None) == 0
    # query rows but no keys at all still need q and out, not the latent inputs
    nokeys = np.array([0, 0], dtype=np.int32)
    assert call(kvp=nokeys.ctypes.data, q=None) == 1


def test_partition_pairs_light_and_equal_tiles():
    # causal, like sequences: 300 tokens = tiles seeing 128, 256, 300 keys
    # (one pair of the first two, one single); 260 = tiles of 128, 256, 260
    # keys (the same); 384 = 128, 256, 384 (the same)
    lens = [300, 260, 384]
    qo = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    items, info = _check_plan(qo, qo, 2, True)
    assert info["items_per_workgroup"] == 2
    pairs = {0: 0, 1: 0, 2: 0}
    singles = {0: 0, 1: 0, 2: 0}
    for w in range(len(items) // 2):
        a, b = items[2 * w], items[2 * w + 1]
        if a[1] == 0:
            continue
        seq = _group(qo, a)[0]
        if b[1] > 0:
            pairs[seq] += 1
        else:
            singles[seq] += 1
    assert pairs == {0: 2, 1: 2, 2: 2}           # per sequence over its 2 heads
    assert singles == {0: 2, 1: 2, 2: 2}
    # mixed or long batches keep one tile per workgroup
    for mixed in ([300, 4096, 100], [5000, 5000], [300, 500]):
        q = np.concatenate([[0], np.cumsum(mixed)]).astype(np.int32)
        _, info = _check_plan(q, q, 2, True)
        assert info["items_per_workgroup"] == 1
    # non-causal: 256 queries over 200 keys pair (400 keys); over 4096 keys
    # nothing pairs and the list keeps one entry per workgroup
    short = np.array([0, 256], dtype=np.int32)
    _, info = _check_plan(short, np.array([0, 200], dtype=np.int32), 2, False)
    assert info["items_per_workgroup"] == 2
    _, info = _check_plan(short, np.array([0, 4096], dtype=np.int32), 2, False)
    assert info["items_per_workgroup"] == 1
    # non-causal sequences whose tiles all see the same keys pair their
    # neighbours from 8 tiles over at most 4096 keys on
    for q_len, k_len, paired in [(1024, 4096, True), (1000, 4096, True), (896, 4096, False),
                                 (1024, 4097, False), (2048, 100, True)]:
        qo1 = np.array([0, q_len], dtype=np.int32)
        kv1 = np.array([0, k_len], dtype=np.int32)
        items1, info = _check_plan(qo1, kv1, 2, False)
        assert info["items_per_workgroup"] == (2 if paired else 1)
        if paired:
            n_tiles = -(-q_len // 128)
            n_pairs = sum(1 for w in range(len(items1) // 2) if items1[2 * w + 1][1] > 0)
            assert n_pairs == 2 * (n_tiles // 2)     # over 2 heads
    # rows that see no key (queries past the keys): their empty tiles pair
    _, info = _check_plan(np.array([0, 300], dtype=np.int32), np.array([0, 2], dtype=np.int32), 2, True)
    assert info["items_per_workgroup"] == 2
    # fp32 plans and head blocks keep one entry per workgroup
    _, info = _check_plan(qo, qo, 2, True, dtype_name="fp32")
    assert info["items_per_workgroup"] == 1
    _, info = _check_plan(qo, qo, 4, True, heads_per_item=2)
    assert info["items_per_workgroup"] == 1
