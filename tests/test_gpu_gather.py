"""Page gathering bit-exact, through the attention kernel's own load path.

``Plan.debug_gather`` launches the kernel ``run`` launches for the plan (same
task list, tile shape, page-address path, loads, waits and barriers) with the
attention replaced by a copy of every landed K/V tile out of LDS.  Its output
is compared byte for byte with a NumPy gather of the logical rows (key j of
request b at page kv_page_indices[kv_indptr[b] + j // P], slot j % P; PR #362,
Review notes), over NaN-poisoned pools, for every page-address path:

* scalar page ids and SGPR-based direct loads: power-of-two pages holding at
  least one load instruction's rows (512 / D keys; FP8: 64 / (D / 16));
* per-lane fixed slots: smaller power-of-two pages;
* per-key page-table lookup with a multiply-shift division: other page sizes
  (FP8: pages below the scalar threshold) and pools whose page stride needs
  more than 32 bits;

on the prefill tile (128 rows x 64 keys, 64 x 32 at head_dim 256) and the
short-query tile (16 / 32 rows x 128 keys), NHD and HND strides, split chunks,
causal and windowed bands, and the full-size workloads.  Keys no task of the
plan loads must be left untouched (the outputs are pre-filled with a sentinel).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import device_inputs, require_gpu, torch_dtype

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FFF   # a NaN pattern in both bf16 and fp16, never a gathered value


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _np_gather(w, pool):
    """Logical rows [sum kv_len, Hkv, D] of every request, in request order."""
    rows = []
    for b in range(w.batch_size):
        first = int(w.kv_indptr[b])
        for j in range(int(w.kv_lens[b])):
            rows.append(pool[int(w.kv_page_indices[first + j // w.page_size]), j % w.page_size])
    if not rows:
        return np.zeros((0, w.num_kv_heads, w.head_dim), pool.dtype)
    return np.stack(rows)


def _covered(p, w):
    """[sum kv_len, Hkv] booleans: keys some task of the plan loads for that kv
    head (task keys [tile_begin, kv_end))."""
    starts = np.concatenate([[0], np.cumsum(np.asarray(w.kv_lens, np.int64))])
    cov = np.zeros((int(starts[-1]), w.num_kv_heads), bool)
    for (b, kvh, _row0, nrows, _lo, end, _slot, tb) in p.work_items():
        if nrows > 0 and end > tb:
            cov[starts[b] + tb:starts[b] + end, kvh] = True
    return cov


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _check(pk, w, p, k, v, want_k, want_v, what, layout="NHD", full=False):
    """want_*: expected logical rows as uint16 bit patterns [sum kv_len, Hkv, D]."""
    total = p.info["total_kv_len"]
    assert total == int(np.sum(w.kv_lens))
    dt = torch_dtype(w.dtype)
    fill = lambda: torch.full((total, w.num_kv_heads, w.head_dim), SENTINEL, dtype=torch.int16,
                              device="cuda").view(dt)
    ko, vo = p.debug_gather(k, v, kv_layout=layout, k_out=fill(), v_out=fill())
    torch.cuda.synchronize()
    gk, gv = _bits(ko), _bits(vo)
    cov = _covered(p, w)
    if full:   # no window: every key of a request with query rows is loaded
        starts = np.concatenate([[0], np.cumsum(np.asarray(w.kv_lens, np.int64))])
        for b in range(w.batch_size):
            if int(w.qo_lens[b]) > 0:
                assert cov[starts[b]:starts[b + 1]].all(), f"{what}: request {b} not all loaded"
    assert cov.any(), f"{what}: vacuous"
    for name, got, want in (("K", gk, want_k), ("V", gv, want_v)):
        assert np.array_equal(got[cov], want[cov]), \
            f"{what}: {name} rows differ at {np.argwhere((got != want).any(-1) & cov)[:5]}"
        assert (got[~cov] == SENTINEL).all(), f"{what}: {name} rows written outside the plan"


def _pool_bits(w, pool):
    return _np_gather(w, pool).view(np.uint16)


# ---------------------------------------------------------------------------
# every page-address path, both tiles, NHD / HND, chunks, bands
# ---------------------------------------------------------------------------
CASES = []
for d in (64, 128, 256):
    for page in (1, 2, 3, 4, 8, 16, 64, 1024):
        for tile in ((1,) if d == 256 else (1, 2)):
            CASES.append((d, page, tile))


@pytest.mark.parametrize("d,page,tile", CASES)
def test_gather_page_paths(pk, d, page, tile):
    rng = np.random.default_rng(d * 100000 + page * 10 + tile)
    qo = [1, 9, 40, 0, 3]
    kv = [1, 70, 300, 5, 129]
    dtype = W.FP16 if d == 64 else W.BF16
    for causal, wl, chunks, layout in ((False, -1, 0, "NHD"), (True, -1, 3, "HND"),
                                       (True, 50, 0, "NHD"), (False, 20, 2, "HND")):
        w = W.build("gather", qo, kv, 8, 2, d, page, causal, wl, dtype,
                    seed=int(rng.integers(1 << 30)), poison=True)
        q, k, v = device_inputs(w)
        p = pk.plan(**w.plan_args(), dtype=torch_dtype(dtype), tile=tile, num_kv_chunks=chunks)
        if layout == "HND":   # the same pool stored [pages, heads, page_size, dim]
            k = k.permute(0, 2, 1, 3).contiguous()
            v = v.permute(0, 2, 1, 3).contiguous()
        _check(pk, w, p, k, v, _pool_bits(w, w.k_pool), _pool_bits(w, w.v_pool),
               f"d={d} P={page} tile={tile} causal={causal} w={wl} chunks={chunks} {layout}",
               layout=layout, full=(wl == -1))


def test_gather_identity_and_single_page(pk):
    """Contiguous KV: an identity table of 8 pages of 16, and the same 128 keys
    as one page of 128."""
    w16 = W.config1(page_size=16, poison=True)
    assert list(w16.kv_page_indices) == list(range(8))
    pool = lambda x: np.ascontiguousarray(x[:8].reshape(1, 128, *x.shape[2:]))
    w128 = W.Workload(**{**w16.__dict__, "page_size": 128, "num_pages": 1,
                         "kv_indptr": np.array([0, 1], np.int32),
                         "kv_page_indices": np.array([0], np.int32),
                         "kv_last_page_len": np.array([128], np.int32),
                         "k_pool": pool(w16.k_pool), "v_pool": pool(w16.v_pool)})
    for w in (w16, w128):
        q, k, v = device_inputs(w)
        for tile in (1, 2):
            p = pk.plan(**w.plan_args(), dtype=torch.float16, tile=tile)
            _check(pk, w, p, k, v, _pool_bits(w, w.k_pool), _pool_bits(w, w.v_pool),
                   f"config1 page {w.page_size} tile={tile}", full=True)


def test_gather_pool_beyond_4_gib(pk):
    """Page offsets past 2^32 bytes (the general per-key path): used pages at
    both ends of a > 4 GiB pool, both tiles."""
    page = 16
    w = W.build("bigpool", [5, 40, 4], [300, 90, 517], 8, 2, 128, page, False, -1, W.BF16,
                seed=78, poison=True)
    _, k_small, v_small = device_inputs(w)
    page_bytes = page * 2 * 128 * 2
    big = (4 << 30) // page_bytes + 4096
    n = w.num_pages
    far = np.arange(n) % 2 == 1
    remap = np.where(far, big - 1 - np.arange(n), np.arange(n)).astype(np.int64)
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
            p = pk.plan(**a, dtype=torch.bfloat16, tile=tile)
            _check(pk, w, p, k, v, _pool_bits(w, w.k_pool), _pool_bits(w, w.v_pool),
                   f"pool of {big} pages tile={tile}", full=True)
    finally:
        del k, v
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# full-size workloads in the launch configuration run() uses
# ---------------------------------------------------------------------------
FULL = [("config2", lambda: W.config2(poison=True), {}),
        ("config2_w127", lambda: W.config2(window_left=127, poison=True), {}),
        ("config3_p1024", lambda: W.config3(window_left=-1, page_size=1024, poison=True), {}),
        ("config3_p1024_w31", lambda: W.config3(window_left=31, page_size=1024, poison=True), {}),
        ("config3_p16_w127", lambda: W.config3(window_left=127, page_size=16, poison=True), {}),
        ("config4_b16_hkv8", lambda: W.config4(batch=16, num_kv_heads=8, poison=True), {}),
        ("config4_b64_hkv4", lambda: W.config4(batch=64, num_kv_heads=4, poison=True), {}),
        ("config5_q64_8chunks", lambda: W.config5(qo_len=64, poison=True),
         {"num_kv_chunks": W.CONFIG5_CHUNKS}),
        ("config5_q1_w4095_8chunks", lambda: W.config5(qo_len=1, window_left=4095, poison=True),
         {"num_kv_chunks": W.CONFIG5_CHUNKS})]


@pytest.mark.parametrize("name,make,opts", FULL, ids=[c[0] for c in FULL])
def test_gather_full_size(pk, name, make, opts):
    w = make()
    q, k, v = device_inputs(w)
    p = pk.plan(**w.plan_args(), dtype=torch_dtype(w.dtype), **opts)
    _check(pk, w, p, k, v, _pool_bits(w, w.k_pool), _pool_bits(w, w.v_pool), name,
           full=(w.window_left == -1))


# ---------------------------------------------------------------------------
# FP8 E4M3 caches: codes loaded through registers, converted into LDS
# ---------------------------------------------------------------------------
def _decoded_bits(w, codes):
    vals = oracle.decode_e4m3(_np_gather(w, codes)).astype(np.float32)   # exact in bf16 / fp16
    if w.dtype == W.BF16:
        return W.round_float32_to_bf16_bits(vals).view(np.uint16)
    return vals.astype(np.float16).view(np.uint16)


FP8_CASES = [(d, page, tile) for d in (64, 128, 256) for page in (1, 3, 4, 8, 16, 256)
             for tile in ((1,) if d == 256 else (1, 2))]


@pytest.mark.parametrize("d,page,tile", FP8_CASES)
def test_gather_fp8_page_paths(pk, d, page, tile):
    rng = np.random.default_rng(7 * d + page * 3 + tile)
    for causal, wl, chunks in ((False, -1, 0), (True, 30, 3)):
        for dtype in (W.BF16, W.FP16):
            w = W.build("gather8", [2, 33, 7], [60, 200, 7], 8, 2, d, page, causal, wl, dtype,
                        seed=int(rng.integers(1 << 30)))
            kc, vc = W.e4m3_pools(w, int(rng.integers(1 << 30)), 0.5, 2.0, poison=True)
            p = pk.plan(**w.plan_args(), dtype=torch_dtype(dtype), tile=tile,
                        num_kv_chunks=chunks, kv_dtype="fp8_e4m3", k_scale=0.5, v_scale=2.0)
            k = torch.from_numpy(kc).cuda()
            v = torch.from_numpy(vc).cuda()
            _check(pk, w, p, k, v, _decoded_bits(w, kc), _decoded_bits(w, vc),
                   f"fp8 d={d} P={page} tile={tile} causal={causal} w={wl} {dtype}",
                   full=(wl == -1))


def test_gather_fp8_full_size(pk):
    w = W.config4(batch=64, num_kv_heads=8, values=True)
    kc, vc = W.e4m3_pools(w, 99, 0.5, 2.0, poison=True)
    p = pk.plan(**w.plan_args(), dtype=torch.bfloat16, kv_dtype="fp8_e4m3", k_scale=0.5,
                v_scale=2.0)
    _check(pk, w, p, torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(),
           _decoded_bits(w, kc), _decoded_bits(w, vc), "fp8 verify B64", full=True)
