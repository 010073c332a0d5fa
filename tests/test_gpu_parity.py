"""GPU parity: the HIP library against the float64 oracle on the same seeded inputs.

Tolerances: max |do| <= 1e-2 (fp16) / 2e-2 (bf16), |dlse| <= 1e-3 (page
gathering is checked bit for bit in test_gpu_gather.py).  Every output
element is compared, at the full sizes of the benchmark workloads too, in the
launch configuration the benchmark uses.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (assert_close, check_full, device_inputs, oracle_full, plan_for,
                      require_gpu, run, to_device, torch_dtype)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _tiny(rng, qo_lens, kv_lens, hq, hkv, d, page, causal, w, dtype, poison=True, seed=0):
    return W.build("tiny", qo_lens, kv_lens, hq, hkv, d, page, causal, w, dtype, seed=seed,
                   poison=poison)


# ---------------------------------------------------------------------------
# config 1: single request, contiguous KV, fp16
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("window_left", [-1, 31])
def test_config1_single_contiguous(pk, window_left):
    """Contiguous KV two ways over the same values: an identity table of 8 pages
    of 16, and the same 128 keys as one page of 128."""
    w16 = W.config1(window_left=window_left, page_size=16, poison=True)
    assert list(w16.kv_page_indices) == list(range(8))
    pool = lambda x: np.ascontiguousarray(x[:8].reshape(1, 128, *x.shape[2:]))
    w128 = W.Workload(**{**w16.__dict__, "page_size": 128, "num_pages": 1,
                         "kv_indptr": np.array([0, 1], np.int32),
                         "kv_page_indices": np.array([0], np.int32),
                         "kv_last_page_len": np.array([128], np.int32),
                         "k_pool": pool(w16.k_pool), "v_pool": pool(w16.v_pool)})
    ref_o, ref_lse = oracle_full(w16)
    ref128 = oracle_full(w128)
    assert np.array_equal(ref_o, ref128[0]) and np.array_equal(ref_lse, ref128[1])
    results = []
    for w in (w16, w128):
        o, lse, _ = run(pk, w)
        assert_close(o, lse, ref_o, ref_lse, w.dtype, f"config1 P={w.page_size} w={window_left}")
        results.append((o, lse))
    assert np.abs(results[0][0] - results[1][0]).max() <= 1e-2


# ---------------------------------------------------------------------------
# tiny exhaustive grid: pages, heads, masks, tiles, dtypes, head dims
# ---------------------------------------------------------------------------
GRID = []
for d in (64, 128):
    for dtype in (W.BF16, W.FP16):
        for (hq, hkv) in ((1, 1), (4, 2), (6, 3), (8, 1)):
            for page in (1, 3, 16):
                GRID.append((d, dtype, hq, hkv, page))


@pytest.mark.parametrize("d,dtype,hq,hkv,page", GRID)
def test_tiny_grid(pk, d, dtype, hq, hkv, page):
    rng = np.random.default_rng(zlib.crc32(repr((d, dtype, hq, hkv, page)).encode()))
    B = int(rng.integers(1, 4))
    qo = rng.integers(1, 40, size=B)
    kv = qo + rng.integers(0, 150, size=B)
    L = int(kv.max())
    for causal in (True, False):
        for w in sorted({-1, 0, 1, 7, L - 2, L - 1, L + 5}):
            wl = _tiny(rng, qo, kv, hq, hkv, d, page, causal, w, dtype,
                       seed=int(rng.integers(1 << 30)))
            ref_o, ref_lse = oracle_full(wl)
            tensors = device_inputs(wl)
            for tile in (1, 2):
                o, lse, _ = run(pk, wl, tensors, tile=tile)
                assert_close(o, lse, ref_o, ref_lse, dtype,
                             f"grid d={d} {dtype} h={hq}/{hkv} P={page} causal={causal} w={w} "
                             f"tile={tile}")


def test_ragged_tails_and_empty_requests(pk):
    # requests with no query rows, one row, and lengths just past tile edges
    qo = [0, 1, 33, 0, 129, 17]
    kv = [5, 64, 65, 0, 129, 300]
    for tile in (0, 1, 2):
        w = W.build("ragged", qo, kv, 8, 2, 128, 16, True, -1, W.BF16, seed=7, poison=True)
        o, lse, _ = run(pk, w, tile=tile)
        ref_o, ref_lse = oracle_full(w)
        assert_close(o, lse, ref_o, ref_lse, w.dtype, f"ragged tile={tile}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("page", [4, 8, 32, 64, 128, 1024])
def test_prefill_kernels_across_page_sizes(pk, d, page):
    """Both tile shapes over every power-of-two page address path (pages that
    hold part of a load instruction's rows, a few instructions' rows, several
    pages per key tile, one page per tile), key runs of one, two, three and
    many tiles, ragged tails, windows, and split chunks writing partials."""
    rng = np.random.default_rng(page * 1000 + d)
    qo = [1, 20, 50, 130, 3]
    kv = [1, 45, 96, 700, 33]
    for causal, w in ((True, -1), (True, 40), (False, 17), (False, -1)):
        wl = W.build("pages", qo, kv, 8, 2, d, page, causal, w, W.BF16,
                     seed=int(rng.integers(1 << 30)), poison=True)
        ref_o, ref_lse = oracle_full(wl)
        tensors = device_inputs(wl)
        for tile in (1, 2):
            for chunks in (0, 3):
                o, lse, _ = run(pk, wl, tensors, tile=tile, num_kv_chunks=chunks)
                assert_close(o, lse, ref_o, ref_lse, wl.dtype,
                             f"pages P={page} d={d} causal={causal} w={w} tile={tile} "
                             f"chunks={chunks}")


@pytest.mark.parametrize("page", [16, 3])
def test_pages_beyond_4_gib_of_pool(pk, page):
    """K/V pools larger than 4 GiB (an unreferenced NaN fill) with the used pages
    scattered over both ends, so page offsets need more than 32 bits: both tile
    shapes, the scalar (page 16) and per-lane (page 3) page-id paths, split chunks."""
    w = W.build("bigpool", [5, 40, 4, 4], [300, 90, 517, 6], 8, 2, 128, page, True, -1, W.BF16,
                seed=77, poison=True)
    ref_o, ref_lse = oracle_full(w)
    q, k_small, v_small = device_inputs(w)
    page_bytes = page * 2 * 128 * 2
    big = (4 << 30) // page_bytes + 4096                      # pool > 4 GiB per tensor
    n = w.num_pages
    far = np.arange(n) % 2 == 1                               # odd pages at the far end
    remap = np.where(far, big - 1 - np.arange(n), np.arange(n)).astype(np.int64)
    assert remap.max() * page_bytes >= (1 << 32)
    idx = torch.from_numpy(remap).cuda()
    k = torch.full((big, page, 2, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    v = torch.full_like(k, float("nan"))
    k[idx] = k_small
    v[idx] = v_small
    del k_small, v_small
    a = w.plan_args()
    a["kv_page_indices"] = remap[w.kv_page_indices].astype(np.int32)
    try:
        for tile in (1, 2):
            for chunks in (0, 3):
                p = pk.plan(**a, dtype=torch.bfloat16, tile=tile, num_kv_chunks=chunks)
                o, lse = p.run(q, k, v)
                torch.cuda.synchronize()
                assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_lse, w.dtype,
                             f"pool of {big} pages of {page} tile={tile} chunks={chunks}")
    finally:
        del k, v
        torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [64, 128, 256])
def test_prefill_row_tiles_with_padding_waves(pk, d):
    """Last row tiles of every fill level: the prefill tile's waves that hold
    only padding rows take their load-and-barrier loop and exit, and the rows
    of the other waves (including a wave's partly filled 16-row blocks) must
    still be exact.  Packed rows per (request, kv head) = 4 * qo_len:
    4, 16, 36, 68, 100, 132 and 260 over 128-row tiles (64-row at head_dim 256),
    with causal, windowed and non-causal masks and split chunks."""
    rng = np.random.default_rng(4242 + d)
    qo = [1, 4, 9, 17, 25, 33, 65]
    kv = [q + int(rng.integers(0, 300)) for q in qo]
    dtype = W.FP16 if d == 64 else W.BF16
    for causal, w in ((True, -1), (True, 23), (False, 50)):
        wl = W.build("padding_waves", qo, kv, 8, 2, d, 16, causal, w, dtype,
                     seed=int(rng.integers(1 << 30)), poison=True)
        ref_o, ref_lse = oracle_full(wl)
        tensors = device_inputs(wl)
        for chunks in (0, 2):
            o, lse, p = run(pk, wl, tensors, tile=1, num_kv_chunks=chunks)
            assert p.info["tile_rows"] == (64 if d == 256 else 128)
            assert_close(o, lse, ref_o, ref_lse, wl.dtype,
                         f"padding waves d={d} causal={causal} w={w} chunks={chunks}")


def test_empty_batch(pk):
    p = pk.plan([0], [0], [], [], 4, 2, 64, 16, True, dtype=torch.float16)
    q = torch.zeros((0, 4, 64), dtype=torch.float16, device="cuda")
    k = torch.zeros((1, 16, 2, 64), dtype=torch.float16, device="cuda")
    o, lse = p.run(q, k, k)
    assert o.shape == (0, 4, 64) and lse.shape == (0, 4)


# ---------------------------------------------------------------------------
# config 2: paged batch prefill (full size, every output element)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("window_left", [-1, 127])
def test_config2_paged_prefill(pk, window_left):
    w = W.config2(window_left=window_left, poison=True)
    o, lse, p = run(pk, w)
    assert p.info["tile_rows"] == 128
    check_full(w, o, lse, f"config2 w={window_left}")


@pytest.mark.parametrize("d,page,dtype", [(64, 48, W.FP16), (128, 2, W.BF16)])
@pytest.mark.parametrize("window_left", [-1, 127])
def test_paged_batch_other_page_paths(pk, d, page, dtype, window_left):
    """The paged batch's lengths (8 requests, qo 128-1024, kv = qo + 0-2048,
    Hq 32 / Hkv 8, causal) on the prefill tile's two other page-address
    paths, at full size: 48-key pages (any page size: a page-table lookup
    per key row and a multiply-shift division) and 2-key pages (power-of-two
    pages shorter than one load instruction's rows: a fixed slot per lane);
    every output element against the oracle over NaN-poisoned pools."""
    rng = np.random.default_rng(2000 + d + page)
    qo = rng.integers(128, 1024, size=8, endpoint=True)
    kv = qo + rng.integers(0, 2048, size=8, endpoint=True)
    w = W.build("paged_batch_pages", qo, kv, 32, 8, d, page, True, window_left, dtype,
                seed=None, rng=rng, poison=True)
    o, lse, p = run(pk, w)
    assert p.info["tile_rows"] == 128
    check_full(w, o, lse, f"paged batch d={d} page={page} window={window_left}")


@pytest.mark.parametrize("d,page,dtype", [(64, 48, W.FP16), (128, 2, W.BF16)])
def test_verify_other_page_paths(pk, d, page, dtype):
    """Verify batch 16 / Hkv 8 (4 queries per request, kv 512-8192, causal)
    on the short-query tile's other page paths, at full size: 48-key pages
    (a page-table lookup per key row) and 2-key pages (a fixed slot per
    lane), where Q is loaded into registers instead of through LDS and the
    split chunks are merged; every output element against the oracle over
    NaN-poisoned pools."""
    rng = np.random.default_rng(4000 + d + page)
    kv = rng.integers(512, 8192, size=16, endpoint=True)
    w = W.build("verify_pages", [4] * 16, kv, 32, 8, d, page, True, -1, dtype, seed=None,
                rng=rng, poison=True)
    o, lse, p = run(pk, w)
    assert p.info["tile_rows"] == 16 and p.info["num_merge_items"] > 0
    check_full(w, o, lse, f"verify d={d} page={page}")


# ---------------------------------------------------------------------------
# config 3: non-causal sliding window, page 1024 and 16
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("page_size", [1024, 16])
def test_config3_noncausal_window(pk, page_size):
    outs = {}
    base = W.config3(window_left=0, page_size=page_size, poison=True)
    tensors = device_inputs(base)
    for wl in (0, 31, 127, 8192, -1):
        w = base.with_window(wl)
        o, lse, _ = run(pk, w, tensors)
        outs[wl] = (o, lse)
        if wl != -1:
            check_full(w, o, lse, f"config3 P={page_size} w={wl}")
    # a window wider than the sequence is the unwindowed result, bit for bit
    assert np.array_equal(outs[8192][0], outs[-1][0])
    assert np.array_equal(outs[8192][1], outs[-1][1])
    assert np.abs(outs[0][0] - outs[-1][0]).max() > 0.1   # non-vacuous


# ---------------------------------------------------------------------------
# config 4: speculative verify
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("batch", [4, 16, 64])
@pytest.mark.parametrize("num_kv_heads", [4, 8])
def test_config4_verify(pk, batch, num_kv_heads):
    w = W.config4(batch=batch, num_kv_heads=num_kv_heads, poison=True)
    q, k, v = device_inputs(w)
    p = pk.verify_plan(w.kv_indptr, w.kv_page_indices, w.kv_last_page_len, 4, w.num_qo_heads,
                       w.num_kv_heads, w.head_dim, w.page_size, dtype=torch.bfloat16)
    o, lse = p.run(q, k, v)
    # the verify wrapper is exactly a causal prefill over a stride-4 qo_indptr
    o2, lse2, _ = run(pk, w, (q, k, v))
    assert np.array_equal(o.float().cpu().numpy(), o2)
    check_full(w, o2, lse2, f"config4 B={batch} Hkv={num_kv_heads}")


# ---------------------------------------------------------------------------
# config 5: long context, KV split into 8 chunks and merged
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("qo_len", [1, 64])
@pytest.mark.parametrize("window_left", [-1, 4095])
def test_config5_split_kv(pk, qo_len, window_left):
    w = W.config5(qo_len=qo_len, window_left=window_left, poison=True)
    tensors = device_inputs(w)
    o8, lse8, p8 = run(pk, w, tensors, num_kv_chunks=W.CONFIG5_CHUNKS)
    # with the 4095-key window every visible key lies in the last 8192-key chunk:
    # the empty chunks are dropped (that chunk may still be sub-split for parallelism)
    chunk = 65536 // W.CONFIG5_CHUNKS
    work = p8.work_items()
    live = work[work[:, 3] > 0]
    if window_left == -1:
        assert p8.info["num_merge_items"] > 0 and (live[:, 4] < chunk).any()
    else:
        assert (live[:, 4] >= (W.CONFIG5_CHUNKS - 1) * chunk).all()
    ref = check_full(w, o8, lse8, f"config5 q={qo_len} w={window_left}")
    oa, lsea, _ = run(pk, w, tensors)   # scheduler's own split
    assert np.abs(oa - o8).max() <= 2e-2
    assert np.abs(lsea - lse8).max() <= 1e-3
    # the same 8 chunks as separate partial states, folded with merge_states
    q, k, v = tensors
    acc_o = acc_l = None
    for c in range(W.CONFIG5_CHUNKS):
        p = plan_for(pk, w, kv_begin=c * chunk, kv_end=(c + 1) * chunk)
        po = torch.empty((w.total_q, w.num_qo_heads, w.head_dim), dtype=torch.float32,
                         device="cuda")
        pb, pl = p.run(q, k, v)
        po.copy_(pb.float())
        if acc_o is None:
            acc_o, acc_l = po, pl
        else:
            acc_o, acc_l = pk.merge_states(acc_o, acc_l, po, pl)
    torch.cuda.synchronize()
    mo, ml = acc_o.cpu().numpy(), acc_l.cpu().numpy()
    assert np.abs(mo - o8).max() <= 2e-2
    assert np.abs(ml - lse8).max() <= 1e-3
    check_full(w, mo, ml, "config5 merge_states fold", ref=ref)


# ---------------------------------------------------------------------------
# invariants on the GPU
# ---------------------------------------------------------------------------
def test_page_relabelling_bitwise(pk):
    w = W.build("relabel", [40, 100], [300, 180], 8, 2, 128, 16, True, 50, W.BF16, seed=10)
    o1, l1, _ = run(pk, w)
    rng = np.random.default_rng(11)
    perm = rng.permutation(w.num_pages)
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    w2 = W.Workload(**{**w.__dict__, "kv_page_indices": perm[w.kv_page_indices].astype(np.int32),
                       "k_pool": k2, "v_pool": v2})
    o2, l2, _ = run(pk, w2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_closed_forms_on_gpu(pk):
    # K = 0: lse_i = log(number of visible keys), o_i = mean of the visible V rows
    w = W.build("kzero", [5, 64], [23, 200], 8, 2, 128, 16, True, 9, W.BF16, seed=12)
    w.k_pool[:] = 0
    o, lse, _ = run(pk, w)
    ref_o, ref_lse = oracle_full(w)
    assert_close(o, lse, ref_o, ref_lse, w.dtype, "K=0")
    for b in range(2):
        Q, L = int(w.qo_lens[b]), int(w.kv_lens[b])
        for i in range(Q):
            lo = max(0, L + i - Q - 9)
            hi = i + L - Q
            r = int(w.qo_indptr[b]) + i
            assert np.abs(lse[r] - np.log(hi - lo + 1)).max() <= 1e-3
    # V = 1: every softmax row sums to one
    w = W.build("vone", [7, 33], [40, 90], 4, 4, 64, 3, False, 20, W.FP16, seed=13)
    w.v_pool[:] = np.float16(1.0)
    o, _, _ = run(pk, w)
    assert np.abs(o - 1.0).max() <= 1e-2


def test_gqa_equals_replicated_heads(pk):
    w = W.build("gqa", [17, 30], [60, 33], 8, 2, 64, 16, True, -1, W.BF16, seed=14)
    o1, l1, _ = run(pk, w)
    rep = W.Workload(**{**w.__dict__, "num_kv_heads": 8,
                        "k_pool": np.repeat(w.k_pool, 4, axis=2),
                        "v_pool": np.repeat(w.v_pool, 4, axis=2)})
    o2, l2, _ = run(pk, rep)
    assert np.abs(o1 - o2).max() <= 2e-2 and np.abs(l1 - l2).max() <= 1e-3


def test_split_equals_unsplit(pk):
    w = W.build("split", [3, 70, 1], [5000, 3000, 900], 16, 4, 128, 16, True, -1, W.BF16,
                seed=15, poison=True)
    ref_o, ref_lse = oracle_full(w)
    for chunks in (0, 1, 2, 3, 8):
        for tile in (1, 2):
            o, lse, p = run(pk, w, num_kv_chunks=chunks, tile=tile)
            assert_close(o, lse, ref_o, ref_lse, w.dtype, f"chunks={chunks} tile={tile}")


@pytest.mark.parametrize("case", ["prefill_d128", "prefill_d64", "short16", "short32", "d256",
                                  "many_slots"])
def test_split_tiles_merged_in_every_run(pk, case):
    """One plan with split query tiles on every tile shape (and up to 24
    partial slots per tile), run three times with fresh values each time,
    every output element against the oracle: each run must merge its own
    partials (a merge reading the previous run's slots, or one that misses
    a slot, shows up as a mismatch)."""
    d, tile, hq, opts = {"prefill_d128": (128, 1, 16, dict(num_kv_chunks=3)),
                         "prefill_d64": (64, 1, 16, dict(num_kv_chunks=5)),
                         "short16": (128, 2, 4, dict(num_kv_chunks=4)),
                         "short32": (128, 2, 16, dict(split_tiles=2)),
                         "d256": (256, 1, 8, dict(num_kv_chunks=4)),
                         "many_slots": (64, 2, 16, dict(split_tiles=1))}[case]
    qo = [1, 4, 7, 16 if case == "short16" else 40, 0, 2]
    kv = [900, 2500, 1300, 3000, 50, 3]
    base = W.build("merge_runs", qo, kv, hq, 4, d, 16, True, -1, W.BF16, seed=31, values=False)
    p = plan_for(pk, base, tile=tile, **opts)
    assert p.info["num_merge_items"] > 0
    assert p.info["tile_rows"] == {"short16": 16, "short32": 32, "many_slots": 32,
                                   "d256": 64}.get(case, 128)
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    pool = (base.num_pages, base.page_size, base.num_kv_heads, d)
    for run_i in range(3):
        w = W.Workload(**{**base.__dict__,
                          "q": W.draw_values(rng, (base.total_q, hq, d), W.BF16),
                          "k_pool": W.draw_values(rng, pool, W.BF16),
                          "v_pool": W.draw_values(rng, pool, W.BF16)})
        o, lse = p.run(*device_inputs(w))
        torch.cuda.synchronize()
        check_full(w, o.float().cpu().numpy(), lse.cpu().numpy(), f"{case} run {run_i}")


@pytest.mark.parametrize("window_left", [-1, 4095])
def test_million_key_context(pk, window_left):
    """One request with 2^20 + 37 keys (65,539 pages of 16 in a permuted pool
    1.5 times that size, ragged last page) and 4 query rows, Hq 8 / Hkv 1,
    D 64: key positions, page ids and page-table offsets far beyond those of
    the benchmark configurations, split into chunks and merged; every output
    element against the oracle, with NaN in every slot the request does not
    reference."""
    w = W.build("million", [4], [(1 << 20) + 37], 8, 1, 64, 16, True, window_left, W.BF16,
                seed=41, poison=True)
    o, lse, p = run(pk, w)
    if window_left < 0:
        assert p.info["num_merge_items"] > 0
    check_full(w, o, lse, f"million keys, window {window_left}")


@pytest.mark.parametrize("causal,window_left", [(True, 40), (False, -1)])
def test_thousands_of_requests(pk, causal, window_left):
    """2,500 requests of 1-6 query rows over 1-300 keys each on 7-key pages
    (the general page path: a page-table lookup per key with a divisor that
    is not a power of two), Hq 8 / Hkv 2, D 64, fp16: a task list of
    thousands of work groups, most of them taken in the order their groups
    start; every output element against the oracle over NaN-poisoned pools."""
    rng = np.random.default_rng(43)
    qo = rng.integers(1, 7, size=2500)
    kv = qo + rng.integers(0, 295, size=2500)
    w = W.build("many", qo, kv, 8, 2, 64, 7, causal, window_left, W.FP16, seed=None, rng=rng,
                poison=True)
    o, lse, p = run(pk, w)
    assert p.info["num_work_items"] >= 5000
    check_full(w, o, lse, f"2500 requests causal={causal} window={window_left}")


def test_key_range_partial_state(pk):
    w = W.build("range", [6, 40], [100, 70], 4, 2, 128, 16, True, 10, W.BF16, seed=16)
    for a, e in ((0, 30), (30, 64), (64, 101), (90, 95)):
        o, lse, _ = run(pk, w, kv_begin=a, kv_end=e)
        ref_o, ref_lse = oracle_full(w, kv_begin=a, kv_end=e)
        assert_close(o, lse, ref_o, ref_lse, w.dtype, f"range [{a},{e})")


# ---------------------------------------------------------------------------
# merge_states
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_merge_states(pk, dtype):
    rng = np.random.default_rng(17)
    rows, heads, d = 37, 5, 96
    oa = rng.standard_normal((rows, heads, d)).astype(np.float32)
    ob = rng.standard_normal((rows, heads, d)).astype(np.float32)
    la = (rng.standard_normal((rows, heads)) * 3).astype(np.float32)
    lb = (rng.standard_normal((rows, heads)) * 3).astype(np.float32)
    la[0, :] = -np.inf
    lb[1, :] = -np.inf
    la[2, :] = lb[2, :] = -np.inf
    oa[0], ob[1] = 0, 0
    ta, tb = torch.from_numpy(oa).to(dtype).cuda(), torch.from_numpy(ob).to(dtype).cuda()
    tla, tlb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    o, lse = pk.merge_states(ta, tla, tb, tlb)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge_states(ta.float().cpu().numpy(), la, tb.float().cpu().numpy(), lb)
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    assert np.abs(o.float().cpu().numpy() - ref_o).max() <= tol
    got_l = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(got_l[fin] - ref_l[fin]).max() <= 1e-5
    # a -inf side leaves the other state unchanged, exactly
    assert torch.equal(o[1], ta[1]) and torch.equal(lse[1], tla[1])
    # in place
    o2, l2 = pk.merge_states(ta, tla, tb, tlb, out=ta, lse_out=tla)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(l2, lse)


# ---------------------------------------------------------------------------
# refusals at run time
# ---------------------------------------------------------------------------
def test_run_refuses_mismatches(pk):
    w = W.build("refuse", [4, 9], [20, 30], 8, 2, 128, 16, True, -1, W.BF16, seed=18)
    q, k, v = device_inputs(w)
    p = plan_for(pk, w)

    def refused(status, fn):
        with pytest.raises(pk.PkvError) as e:
            fn()
        assert e.value.status_name == status, str(e.value)
        return str(e.value)

    msg = refused("EMISMATCH", lambda: p.run(q[:, :4], k, v))
    assert "planned 8" in msg and "given 4" in msg
    refused("EMISMATCH", lambda: p.run(q[:5], k, v))                       # too few rows
    refused("EMISMATCH", lambda: p.run(q, k[:, :, :1], v))                 # kv heads
    refused("EMISMATCH", lambda: p.run(q, k[:, :8], v[:, :8]))             # page size
    refused("EMISMATCH", lambda: p.run(q.half(), k, v))                    # dtype
    refused("EINVAL", lambda: p.run(q, k[:1], v[:1]))                      # pool too small
    qs = torch.empty((q.shape[0], 8, 256), dtype=q.dtype, device=q.device)[:, :, ::2]
    refused("ELAYOUT", lambda: p.run(qs, k, v))                            # strided head_dim
    # padded q / o are accepted (token counts are minimums) and o rows past the plan untouched
    qp = torch.zeros((q.shape[0] + 5, 8, 128), dtype=q.dtype, device=q.device)
    qp[:q.shape[0]] = q
    out = torch.full((q.shape[0] + 5, 8, 128), 7.0, dtype=q.dtype, device=q.device)
    o, _ = p.run(qp, k, v, out=out)
    o_ref, _ = p.run(q, k, v)
    assert torch.equal(o[:q.shape[0]], o_ref) and torch.all(o[q.shape[0]:] == 7)
    # a strided q (a slice of a fused qkv tensor) is honoured, not refused
    qkv = torch.zeros((q.shape[0], 12, 128), dtype=q.dtype, device=q.device)
    qkv[:, :8] = q
    o_s, _ = p.run(qkv[:, :8], k, v)
    assert torch.equal(o_s, o_ref)
    # lse rows are a minimum too: a short lse is refused by the library, a padded
    # one is filled for the planned rows only
    short = torch.empty((q.shape[0] - 1, 8), dtype=torch.float32, device=q.device)
    assert "lse rows" in refused("EMISMATCH", lambda: p.run(q, k, v, lse=short))
    lp = torch.full((q.shape[0] + 3, 8), 5.0, dtype=torch.float32, device=q.device)
    _, l_pad = p.run(q, k, v, lse=lp)
    _, l_ref = p.run(q, k, v)
    assert torch.equal(l_pad[:q.shape[0]], l_ref) and torch.all(l_pad[q.shape[0]:] == 5)


def test_two_plans_on_two_streams(pk):
    """Runs of different plans may overlap: a verify batch (tasks past the
    first 256 taken in start order from its own counter) and a split-KV
    prefill (merged by its own merge launch), each run five times on its own
    stream with no synchronisation between the two streams, both checked in
    full against the oracle."""
    w1 = W.config4(batch=64, num_kv_heads=8, poison=True)
    w2 = W.build("two_streams", [40, 3, 70], [3000, 900, 2500], 16, 4, 128, 16, True, -1,
                 W.BF16, seed=51, poison=True)
    p1 = plan_for(pk, w1)
    p2 = plan_for(pk, w2, num_kv_chunks=3)
    assert p1.info["num_work_items"] > 256 and p2.info["num_merge_items"] > 0
    t1, t2 = device_inputs(w1), device_inputs(w2)
    torch.cuda.synchronize()    # plans uploaded on the current stream
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(5):
        with torch.cuda.stream(s1):
            o1, l1 = p1.run(*t1)
        with torch.cuda.stream(s2):
            o2, l2 = p2.run(*t2)
    torch.cuda.synchronize()
    check_full(w1, o1.float().cpu().numpy(), l1.cpu().numpy(), "verify on stream 1")
    check_full(w2, o2.float().cpu().numpy(), l2.cpu().numpy(), "split prefill on stream 2")


def test_plan_refused_under_stream_capture(pk):
    """plan uploads its task list from a staging buffer whose reuse is ordered by
    an event, which capture would never record: a runnable plan on a capturing
    stream is refused before any device call, and capture proceeds unharmed."""
    w = W.build("capture", [4, 9], [20, 30], 8, 2, 128, 16, True, -1, W.BF16, seed=19)
    q, k, v = device_inputs(w)
    p = plan_for(pk, w)
    o_ref, l_ref = p.run(q, k, v)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        o = torch.empty_like(o_ref)
        lse = torch.empty_like(l_ref)
        with torch.cuda.graph(g, stream=s):
            with pytest.raises(pk.PkvError, match="capturing"):
                plan_for(pk, w)
            p.run(q, k, v, out=o, lse=lse)          # run() may be captured
    for _ in range(2):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


# ---------------------------------------------------------------------------
# logits soft-cap
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cap", [2.0, 30.0])
@pytest.mark.parametrize("d,dtype", [(64, W.FP16), (128, W.BF16)])
def test_soft_cap_tiny(pk, cap, d, dtype):
    rng = np.random.default_rng(int(cap) * 7 + d)
    qo = [1, 17, 40]
    kv = [30, 17, 200]
    for causal, wl in ((True, -1), (False, 9), (True, 50)):
        # a large sm_scale makes the cap bite on N(0, 1) data
        w = W.build("cap", qo, kv, 8, 2, d, 16, causal, wl, dtype,
                    seed=int(rng.integers(1 << 30)), poison=True, sm_scale=0.5)
        w.logits_soft_cap = cap
        ref_o, ref_lse = oracle_full(w)
        tensors = device_inputs(w)
        for tile in (1, 2):
            o, lse, _ = run(pk, w, tensors, tile=tile)
            assert_close(o, lse, ref_o, ref_lse, dtype,
                         f"cap={cap} d={d} causal={causal} w={wl} tile={tile}")


@pytest.mark.parametrize("cap", [1000.0, 1024.0, 1025.0, 4096.0])
def test_soft_cap_small_logits_both_forms(pk, cap):
    """Logits far below the cap (sm_scale 0.01: |s| ~ 0.1, s / cap ~ 1e-4),
    where tanh(y) = 1 - 2 / (1 + e^{2y}) loses most of y to cancellation:
    caps up to 1024 take that form alone (its error, a few ulp of 1 times
    the cap, stays far inside the tolerances), larger ones its Taylor series
    near 0.  Both on both tile shapes, against the oracle."""
    rng = np.random.default_rng(int(cap))
    w = W.build("capsmall", [1, 17, 40], [30, 17, 200], 8, 2, 128, 16, True, -1, W.BF16,
                seed=int(rng.integers(1 << 30)), poison=True, sm_scale=0.01)
    w.logits_soft_cap = cap
    ref_o, ref_lse = oracle_full(w)
    tensors = device_inputs(w)
    for tile in (1, 2):
        o, lse, _ = run(pk, w, tensors, tile=tile)
        assert_close(o, lse, ref_o, ref_lse, W.BF16, f"cap={cap} tile={tile}")


def test_soft_cap_full_size(pk):
    w = W.config2(poison=True)
    w.logits_soft_cap = 5.0
    w.sm_scale = 0.3
    o, lse, _ = run(pk, w)
    check_full(w, o, lse, "config2 cap 5")
    # a cap far above every logit gives the uncapped result
    w2 = W.config4(batch=16, num_kv_heads=8, poison=True)
    o_a, l_a, _ = run(pk, w2)
    w2.logits_soft_cap = 1e6
    o_b, l_b, _ = run(pk, w2)
    assert np.abs(o_a - o_b).max() <= 1e-2 and np.abs(l_a - l_b).max() <= 1e-3


# ---------------------------------------------------------------------------
# head_dim 256 (prefill tile only: 64 rows x 32 keys)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [W.BF16, W.FP16])
@pytest.mark.parametrize("page", [1, 3, 16])
def test_head_dim_256_tiny(pk, dtype, page):
    rng = np.random.default_rng(page * 31 + (dtype == W.BF16))
    for (hq, hkv) in ((4, 2), (8, 1)):
        qo = [int(x) for x in rng.integers(1, 70, size=3)]
        kv = [q + int(x) for q, x in zip(qo, rng.integers(0, 120, size=3))]
        for causal, wl in ((True, -1), (False, 10), (True, 40)):
            w = W.build("d256", qo, kv, hq, hkv, 256, page, causal, wl, dtype,
                        seed=int(rng.integers(1 << 30)), poison=True)
            ref_o, ref_lse = oracle_full(w)
            tensors = device_inputs(w)
            for chunks in (0, 3):
                o, lse, p = run(pk, w, tensors, num_kv_chunks=chunks)
                assert p.info["tile_rows"] == 64 and p.info["tile_keys"] == 32
                assert_close(o, lse, ref_o, ref_lse, dtype,
                             f"d256 P={page} h={hq}/{hkv} causal={causal} w={wl} chunks={chunks}")


def test_head_dim_256_full_size(pk):
    rng = np.random.default_rng(2560)
    qo = rng.integers(128, 1024, size=4, endpoint=True)
    kv = qo + rng.integers(0, 2048, size=4, endpoint=True)
    w = W.build("prefill_d256", qo, kv, 16, 8, 256, 16, True, -1, W.BF16, seed=None, rng=rng,
                poison=True)
    o, lse, _ = run(pk, w)
    check_full(w, o, lse, "d256 prefill")
    w.logits_soft_cap = 50.0
    o, lse, _ = run(pk, w)
    check_full(w, o, lse, "d256 prefill cap 50")
    kv_v = rng.integers(512, 8192, size=16, endpoint=True)
    wv = W.build("verify_d256", [4] * 16, kv_v, 16, 8, 256, 16, True, -1, W.BF16, seed=None,
                 rng=rng, poison=True)
    o, lse, _ = run(pk, wv)
    check_full(wv, o, lse, "d256 verify")
