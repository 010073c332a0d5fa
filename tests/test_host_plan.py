"""Host logic of the C-ABI library, on the CPU (no device call is made):
exported symbols, every plan refusal, and the scheduler's task list."""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_cache_prefill_amd as pk
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "pkv.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", header))
    assert {"pkv_plan", "pkv_run", "pkv_merge_states", "pkv_workspace_size",
            "pkv_plan_destroy", "pkv_last_error"} <= declared
    lib = ctypes.CDLL(pk.library_path(), mode=os.RTLD_NOW)   # every symbol resolvable
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in include/pkv.h but not exported"
    pk.load_library()
    assert b"gfx950" in pk.load_library().pkv_version()


def _base():
    return dict(qo_indptr=[0, 4, 10], kv_indptr=[0, 2, 5], kv_page_indices=[3, 0, 1, 4, 2],
                kv_last_page_len=[5, 16], num_qo_heads=8, num_kv_heads=2, head_dim=128,
                page_size=16, causal=True, window_left=-1)


def refused(status, **over):
    args = {**_base(), **over}
    with pytest.raises(pk.PkvError) as e:
        pk.plan_host(**args)
    assert e.value.status_name == status, str(e.value)
    return str(e.value)


def test_plan_refusals():
    assert pk.plan_host(**_base()).info["num_work_items"] > 0
    assert "given 12" in refused("EGQA", num_qo_heads=12, num_kv_heads=8)
    refused("EGQA", num_qo_heads=4, num_kv_heads=8)
    refused("EGQA", num_kv_heads=0)
    refused("EGQA", num_kv_heads=-2)
    refused("EINVAL", head_dim=96)
    assert pk.plan_host(**{**_base(), "head_dim": 256}).info["tile_rows"] == 64
    assert "head_dim 256" in refused("EINVAL", head_dim=256, tile=2)
    refused("EINVAL", page_size=0)
    refused("EINVAL", window_left=-2)
    refused("EINVAL", qo_indptr=[1, 4, 10])
    refused("EINVAL", kv_indptr=[0, 3, 2], kv_page_indices=[0, 1, 2])
    refused("EINVAL", qo_indptr=[0, 4, 3])
    assert "kv_last_page_len[0]" in refused("EINVAL", kv_last_page_len=[0, 16])
    refused("EINVAL", kv_last_page_len=[17, 16])
    refused("EINVAL", kv_page_indices=[3, 0, -1, 4, 2])
    # causal with kv_len < qo_len: request 0 has 21 keys, give it 30 rows
    msg = refused("EINVAL", qo_indptr=[0, 30, 36])
    assert "request 0" in msg and "kv_len" in msg
    # the same shape is fine without the causal mask
    pk.plan_host(**{**_base(), "qo_indptr": [0, 30, 36], "causal": False})
    # query rows but no key
    refused("EINVAL", kv_indptr=[0, 0, 5], kv_page_indices=[1, 4, 2, 0, 3], causal=False)
    # batch 0 needs 0 rows; indptr / last length mismatch is caught by the binding
    assert pk.plan_host([0], [0], [], [], 4, 2, 64, 16, True).info["num_work_items"] == 0
    refused("EINVAL", kv_last_page_len=[5])
    refused("EINVAL", tile=3)
    refused("EINVAL", num_kv_chunks=-1)
    refused("EINVAL", split_tiles=-1)
    refused("EINVAL", kv_begin=10, kv_end=5)


def test_rejected_plan_leaves_earlier_plan_usable():
    good = pk.plan_host(**_base())
    before = good.work_items().copy()
    with pytest.raises(pk.PkvError):
        pk.plan_host(**{**_base(), "num_qo_heads": 12, "num_kv_heads": 8})
    assert np.array_equal(good.work_items(), before)
    assert good.info["has_device_copy"] == 0


def test_host_plan_cannot_run():
    p = pk.plan_host(**_base())
    with pytest.raises(pk.PkvError) as e:
        p.run(None, None, None)
    assert e.value.status_name == "ENOTPLANNED"


def _visible(i, Q, L, causal, w):
    hi = i + L - Q if causal else L - 1
    lo = 0 if (w == -1) else max(0, L + i - Q - w)
    return lo, min(hi, L - 1)


def check_coverage(w, **opts):
    """Every packed row of every (request, kv head) is in exactly one row tile, and
    the tile's chunks cover each row's visible keys exactly once."""
    args = w.plan_args()
    p = pk.plan_host(**args, **opts)
    items = p.work_items()
    info = p.info
    G = w.num_qo_heads // w.num_kv_heads
    NK = info["tile_keys"]
    kb, ke = opts.get("kv_begin", 0), opts.get("kv_end", -1)
    tiles = {}
    for (b, kvh, row0, nrows, lo, end, slot, tb) in items:
        assert tb % NK == 0 and tb <= max(lo, 0)
        assert nrows <= info["tile_rows"]
        tiles.setdefault((b, kvh, row0, nrows), []).append((lo, end, slot))
    slots = [s for (_, _, _, _, _, _, s, _) in items if s >= 0]
    assert sorted(slots) == list(range(info["num_partial_slots"]))
    for b in range(w.batch_size):
        Q, L = int(w.qo_lens[b]), int(w.kv_lens[b])
        for kvh in range(w.num_kv_heads):
            mine = sorted(t for t in tiles if t[0] == b and t[1] == kvh)
            covered = []
            for (_, _, row0, nrows) in mine:
                covered.extend(range(row0, row0 + nrows))
            assert covered == list(range(Q * G))
            for key in mine:
                chunks = sorted(tiles[key])
                if len(chunks) > 1:
                    assert all(s >= 0 for (_, _, s) in chunks)
                for (a, e_, _), (a2, _, _) in zip(chunks, chunks[1:]):
                    assert e_ <= a2   # disjoint
                _, _, row0, nrows = key
                for r in range(row0, row0 + nrows):
                    lo, hi = _visible(r // G, Q, L, w.causal, w.window_left)
                    lo, hi = max(lo, kb), min(hi, L - 1 if ke < 0 else min(hi, ke - 1))
                    need = set(range(lo, hi + 1))
                    got = set()
                    for (a, e_, _) in chunks:
                        got |= set(range(a, e_)) & need
                    assert got == need, (b, kvh, r)
    return p


@pytest.mark.parametrize("cfg", ["c1", "c2", "c2w", "c3", "c4", "c5", "c5q1w"])
def test_schedule_covers_every_visible_key(cfg):
    w = {"c1": lambda: W.config1(window_left=31, values=False),
         "c2": lambda: W.config2(values=False),
         "c2w": lambda: W.config2(window_left=127, values=False),
         "c3": lambda: W.config3(window_left=31, values=False),
         "c4": lambda: W.config4(batch=4, num_kv_heads=4, values=False),
         "c5": lambda: W.config5(qo_len=64, values=False),
         "c5q1w": lambda: W.config5(qo_len=1, window_left=4095, values=False)}[cfg]()
    if cfg in ("c2", "c3", "c5"):
        # full coverage check is O(rows * keys) in Python: shrink the big ones
        w = W.build(w.name, np.minimum(w.qo_lens, 120), np.minimum(w.kv_lens, 900),
                    w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, w.causal,
                    w.window_left, w.dtype, seed=1, values=False)
    check_coverage(w)
    for opts in ({"num_kv_chunks": 3}, {"tile": 1}, {"tile": 2}, {"kv_begin": 33, "kv_end": 700},
                 {"num_kv_chunks": 8, "tile": 2}, {"split_tiles": 1}, {"split_tiles": 5},
                 {"num_kv_chunks": 3, "split_tiles": 2}):
        check_coverage(w, **opts)


@pytest.mark.parametrize("batch,hkv", [(4, 4), (4, 8), (16, 4), (16, 8), (64, 4), (64, 8)])
def test_split_choice(batch, hkv):
    """Forced chunk sizes give items of at most that many key tiles; the
    automatic choice splits only when tasks are fewer than two per CU, and its
    chunks are never shorter than four key tiles (the short-query tile)."""
    w = W.config4(batch=batch, num_kv_heads=hkv, values=False)
    tasks = batch * hkv
    for st in (3, 8):
        p = pk.plan_host(**w.plan_args(), split_tiles=st)
        it = p.work_items()
        nk = p.info["tile_keys"]
        ntiles = (it[:, 5] - it[:, 7] + nk - 1) // nk
        assert ntiles.max() <= st
    p = pk.plan_host(**w.plan_args())
    it = p.work_items()
    nk = p.info["tile_keys"]
    if tasks >= 512:
        assert len(it) == tasks and p.info["num_merge_items"] == 0
    else:
        split = it[it[:, 6] >= 0]
        # every split chunk but a task's last starts on a multiple of the chunk size
        per_task = {}
        for row in split:
            per_task.setdefault((row[0], row[1], row[2]), []).append(row)
        for rows in per_task.values():
            rows = sorted(rows, key=lambda r: r[4])
            for r in rows[:-1]:
                assert (r[5] - r[7] + nk - 1) // nk >= 4


def test_wide_window_schedules_like_no_window():
    w = W.config2(values=False)
    a = pk.plan_host(**{**w.plan_args(), "window_left": -1}).work_items()
    b = pk.plan_host(**{**w.plan_args(), "window_left": 5000}).work_items()
    assert np.array_equal(a, b)


def test_window_skips_pages():
    w = W.config3(window_left=0, page_size=16, values=False)
    narrow = pk.plan_host(**w.plan_args()).work_items()
    full = pk.plan_host(**{**w.plan_args(), "window_left": -1}).work_items()
    loaded = lambda it: int(np.sum(it[:, 5] - it[:, 7]))
    assert loaded(narrow) * 4 < loaded(full)


def test_forced_chunks_for_long_context():
    w = W.config5(qo_len=64, values=False)
    p = pk.plan_host(**w.plan_args(), num_kv_chunks=8)
    # every query tile is split into the 8 chunks (each maybe sub-split alike)
    n_items, n_merge = p.info["num_work_items"], p.info["num_merge_items"]
    assert n_merge > 0 and n_items % n_merge == 0 and n_items // n_merge >= 8
    it = p.work_items()
    live = it[it[:, 3] > 0]
    # no work item crosses a chunk boundary, and every boundary is an item end
    assert np.all(live[:, 4] // 8192 == (live[:, 5] - 1) // 8192)
    ends = set(live[:, 5].tolist())
    assert all(8192 * c in ends for c in range(1, 9))


def test_verify_plan_is_causal_stride_k():
    w = W.config4(batch=16, num_kv_heads=8, values=False)
    a = pk.plan_host(**w.plan_args()).work_items()
    qo = np.arange(17) * 4
    b = pk.plan_host(qo, w.kv_indptr, w.kv_page_indices, w.kv_last_page_len, 32, 8, 128, 16,
                     True).work_items()
    assert np.array_equal(a, b)


def _append_call(lib, dtype=0, tokens=4, heads=2, dim=128, batch=1, k_page_size=16,
                 v_page_size=16, k_pages=8, v_pages=8, ak_s_tok=256, k_s_tok=256, ptr=None):
    # pointers are never dereferenced: every case here is refused (or empty) on the host
    return lib.pkv_append_kv(ptr, ak_s_tok, 128, ptr, 256, 128, tokens, heads, dim,
                             ptr, ptr, ptr, batch, ptr, 4,
                             ptr, k_pages, k_page_size, 16 * 256, k_s_tok, 128,
                             ptr, v_pages, v_page_size, 16 * 256, 256, 128,
                             dtype, None, None)


def test_append_refusals_on_host():
    lib = pk.load_library()
    assert _append_call(lib, tokens=0) == 0                       # nothing to write
    assert _append_call(lib, dtype=2) == pk.PKV_EINVAL            # fp32 cache
    assert _append_call(lib, dim=100) == pk.PKV_EINVAL
    assert _append_call(lib, heads=0) == pk.PKV_EINVAL
    assert _append_call(lib, tokens=-1) == pk.PKV_EINVAL
    assert _append_call(lib, v_page_size=8) == pk.PKV_EMISMATCH
    assert _append_call(lib, v_pages=9) == pk.PKV_EMISMATCH
    assert _append_call(lib) == pk.PKV_EINVAL                     # NULL device pointers
    assert b"NULL" in lib.pkv_last_error()
    fake = 1 << 20                                                # aligned, never touched
    assert _append_call(lib, ptr=fake, ak_s_tok=260) == pk.PKV_ELAYOUT
    assert _append_call(lib, ptr=fake, k_s_tok=1 << 31) == pk.PKV_ELAYOUT
    assert _append_call(lib, ptr=fake + 8) == pk.PKV_ELAYOUT      # misaligned


def test_custom_mask_refusals_and_plan():
    mats = [W.tree_topology_mask(3, [-1, 0, 0]), W.tree_topology_mask(5, [-1, -1])]
    data, ind = W.pack_custom_mask(mats)
    base = dict(qo_indptr=[0, 3, 5], kv_indptr=[0, 2, 4], kv_page_indices=[0, 1, 2, 3],
                kv_last_page_len=[2, 3], num_qo_heads=8, num_kv_heads=2, head_dim=64,
                page_size=4, causal=False, window_left=-1)
    p = pk.plan_host(**base, custom_mask=data, mask_indptr=ind)
    assert p.info["num_work_items"] > 0
    ib, _ = pk.workspace_size(**base, custom_mask=data, mask_indptr=ind)
    ib0, _ = pk.workspace_size(**base)
    assert ib >= ib0 + len(data)
    with pytest.raises(pk.PkvError, match="causal"):
        pk.plan_host(**{**base, "causal": True}, custom_mask=data, mask_indptr=ind)
    short = ind.copy()
    short[2] -= 1
    with pytest.raises(pk.PkvError, match="request 1 needs"):
        pk.plan_host(**base, custom_mask=data, mask_indptr=short)
    with pytest.raises(pk.PkvError, match="both or neither"):
        pk.plan_host(**base, custom_mask=data)
    bad0 = ind.copy()
    bad0[0] = -1
    with pytest.raises(pk.PkvError, match="mask_indptr"):
        pk.plan_host(**base, custom_mask=data, mask_indptr=bad0)
    # the binding checks both arrays' lengths before the library reads them
    with pytest.raises(pk.PkvError, match="mask_indptr: expected 3 entries"):
        pk.plan_host(**base, custom_mask=data, mask_indptr=ind[:2])
    with pytest.raises(pk.PkvError, match="custom_mask: expected at least"):
        pk.plan_host(**base, custom_mask=data[:-1], mask_indptr=ind)
    # a mask of no bytes (no request has a query row) is a mask, not a missing one
    e_data, e_ind = W.pack_custom_mask([np.zeros((0, 6), bool), np.zeros((0, 7), bool)])
    assert len(e_data) == 0
    p = pk.plan_host(**dict(base, qo_indptr=[0, 0, 0]), custom_mask=e_data, mask_indptr=e_ind)
    assert p.info["total_q_rows"] == 0


def test_sampling_refusals_on_host():
    lib = pk.load_library()
    assert lib.pkv_chain_speculative_sampling_workspace_size(64, 128256) == 64 * 126 * 16
    assert lib.pkv_chain_speculative_sampling_workspace_size(0, 10) == 0
    fake = 1 << 20   # aligned, never dereferenced: every call below is refused on the host
    call = lambda B, n, V, ws, wsb: lib.pkv_chain_speculative_sampling(
        fake, fake, fake, fake, fake, B, n, V, fake, fake, ws, wsb, None)
    assert call(0, 4, 100, None, 0) == 0                               # empty batch
    assert call(-1, 4, 100, fake, 1 << 20) == pk.PKV_EINVAL
    assert call(2, -1, 100, fake, 1 << 20) == pk.PKV_EINVAL
    assert call(2, 4, 0, fake, 1 << 20) == pk.PKV_EINVAL
    assert call(2, 4, (1 << 20) + 1, fake, 1 << 30) == pk.PKV_EINVAL
    assert call(2, 4, 5000, fake, 16) == pk.PKV_EWORKSPACE            # 2 x 5 tiles x 16 B needed
    assert call(2, 4, 5000, None, 1 << 20) == pk.PKV_EWORKSPACE
    assert call(2, 4, 5000, fake + 4, 1 << 20) == pk.PKV_ELAYOUT


# ---------------------------------------------------------------------------
# C-ABI refusals that the Python binding leaves to the library
# ---------------------------------------------------------------------------
def _c_plan_args(num_indices=None, sm_scale=0.125):
    """pkv_plan arguments for _base() as ctypes values (host-only plan)."""
    b = _base()
    arr = lambda x: np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    qo, kv, idx, last = (arr(b["qo_indptr"]), arr(b["kv_indptr"]), arr(b["kv_page_indices"]),
                         arr(b["kv_last_page_len"]))
    p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    n = len(idx) if num_indices is None else num_indices
    keep = (qo, kv, idx, last)
    head = (p32(qo), p32(kv), p32(idx), n, p32(last), 2, b["num_qo_heads"], b["num_kv_heads"],
            b["head_dim"], b["page_size"], 1, -1)
    return keep, head


def _c_plan(num_indices=None, sm_scale=0.125):
    lib = pk.load_library()
    keep, head = _c_plan_args(num_indices)
    h = ctypes.c_void_p()
    st = lib.pkv_plan(*head, ctypes.c_float(sm_scale), pk.PKV_BF16, None, 0, None, 0, None,
                      None, ctypes.byref(h))
    return st, h, lib.pkv_last_error().decode()


def test_c_abi_refuses_page_table_of_wrong_length():
    """num_indices must equal kv_indptr[batch]: a short array would otherwise be
    read past its end, a long one silently truncated (PR #399, What changed:
    inputs the kernels would compute wrongly are refused before any compute)."""
    lib = pk.load_library()
    st, h, _ = _c_plan()
    assert st == pk.PKV_OK and h.value
    lib.pkv_plan_destroy(h)
    for n in (4, 6, 0, -1):
        st, h, msg = _c_plan(num_indices=n)
        assert st == pk.PKV_EINVAL and not h.value, (n, msg)
        assert "num_indices" in msg and f"given {n}" in msg, msg
        if n >= 0:
            assert "kv_indptr[2]=5" in msg, msg
    keep, head = _c_plan_args(num_indices=3)
    ib, fb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.pkv_workspace_size(*head, None, ctypes.byref(ib), ctypes.byref(fb)) == pk.PKV_EINVAL
    assert "num_indices" in lib.pkv_last_error().decode()
    # the binding passes the array's own length: a short or long list is refused too
    for idx in ([3, 0, 1, 4], [3, 0, 1, 4, 2, 5]):
        assert "num_indices" in refused("EINVAL", kv_page_indices=idx)


def test_c_abi_refuses_non_positive_sm_scale():
    """The kernels take each row's maximum before scaling: sm_scale must be > 0."""
    for bad in (0.0, -0.125, float("nan"), float("inf")):
        st, h, msg = _c_plan(sm_scale=bad)
        assert st == pk.PKV_EINVAL and not h.value and "sm_scale" in msg, (bad, msg)
    with pytest.raises(pk.PkvError, match="sm_scale"):
        pk.plan_host(**_base(), sm_scale=-1.0)


def test_c_abi_run_refuses_short_lse_and_rows():
    """pkv_run checks q / o / lse rows (minimums) against the plan before anything
    else; a host-only plan that passes every check is then not runnable.  The
    pointers are never dereferenced: every refusal precedes any device call."""
    lib = pk.load_library()
    p = pk.plan_host(**_base(), dtype="bf16")
    rows = p.info["total_q_rows"]
    assert rows == 10 and p.info["total_kv_len"] == 21 + 48   # (2-1)*16+5, (3-1)*16+16
    fake = 1 << 20   # 16-byte aligned, never read

    def run(q_rows=rows, o_rows=rows, lse=fake, lse_rows=rows):
        st = lib.pkv_run(p._h, fake, q_rows, 8, 128, 8 * 128, 128,
                         fake, 5, 16, 2, 128, 16 * 2 * 128, 2 * 128, 128,
                         fake, 5, 16, 2, 128, 16 * 2 * 128, 2 * 128, 128,
                         pk.PKV_BF16, fake, o_rows, lse, lse_rows, None)
        return st, lib.pkv_last_error().decode()

    st, msg = run(lse_rows=rows - 1)
    assert st == pk.PKV_EMISMATCH and "lse rows" in msg and "given 9" in msg, msg
    st, msg = run(o_rows=rows - 1)
    assert st == pk.PKV_EMISMATCH and "o rows" in msg, msg
    st, msg = run(q_rows=rows - 1)
    assert st == pk.PKV_EMISMATCH and "q rows" in msg, msg
    # padded buffers and a skipped lse are fine (then only host-only-ness refuses)
    for kw in ({"lse_rows": rows + 5, "o_rows": rows + 5, "q_rows": rows + 5},
               {"lse": None, "lse_rows": 0}):
        st, msg = run(**kw)
        assert st == pk.PKV_ENOTPLANNED, msg


def test_binding_computes_nothing_from_the_page_table():
    """total_kv_len (the rows of a debug gather) comes from the library's plan."""
    w = W.build("kvtotal", [3, 0, 5], [40, 17, 33], 4, 2, 64, 16, True, -1, W.BF16, seed=1,
                values=False)
    p = pk.plan_host(**w.plan_args())
    assert p.info["total_kv_len"] == int(np.sum(w.kv_lens))
    assert p.info["num_page_indices"] == len(w.kv_page_indices)


def test_no_alloc_sampling_refuses_sizes_beyond_its_array():
    """The allocation-free sampling entry point holds its tile sums in a 4 MiB
    array per GPU: batch * ceil(vocab / 1024) > 262144 tiles is refused before
    any device call (the pointers are never dereferenced)."""
    lib = pk.load_library()
    fake = 1 << 20
    call = lambda B, V: lib.pkv_chain_speculative_sampling_no_alloc(
        fake, fake, fake, fake, fake, B, 4, V, fake, fake, None)
    assert call(300, 1 << 20) == pk.PKV_EINVAL
    msg = lib.pkv_last_error().decode()
    assert "262144" in msg and "307200" in msg, msg
    assert call(257, 1 << 20) == pk.PKV_EINVAL
    assert call(0, 10) == pk.PKV_OK          # nothing to do
    assert call(4, 0) == pk.PKV_EINVAL      # vocabulary out of range, as for the other entry
