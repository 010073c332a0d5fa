"""Tree-draft verify (custom topology masks) on the GPU against the oracle:
tiny exhaustive cases over page sizes, head dims, dtypes, windows and both
tile shapes; arbitrary (non-tree) masks with fully masked rows; full-size
batches with every output element compared; reductions to the causal path."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_close, check_full, device_inputs, oracle_full, require_gpu, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _tree_workload(rng, trees, prefixes, hq, hkv, d, page, window, dtype, mats=None):
    if mats is None:
        mats = [W.tree_topology_mask(p, W.random_tree_parents(rng, n))
                for n, p in zip(trees, prefixes)]
    qo = [m.shape[0] for m in mats]
    kv = [m.shape[1] for m in mats]
    w = W.build("tree", qo, kv, hq, hkv, d, page, False, window, dtype,
                seed=int(rng.integers(1 << 30)), poison=True)
    w.custom_mask, w.mask_indptr = W.pack_custom_mask(mats)
    return w


GRID = [(d, dtype, page) for d in (64, 128) for dtype in (W.BF16, W.FP16) for page in (1, 3, 16)]


@pytest.mark.parametrize("d,dtype,page", GRID)
def test_tree_tiny_grid(pk, d, dtype, page):
    rng = np.random.default_rng(zlib.crc32(repr((d, dtype, page)).encode()))
    for trial in range(4):
        B = int(rng.integers(1, 4))
        trees = [int(x) for x in rng.integers(1, 10, size=B)]
        prefixes = [int(x) for x in rng.integers(0, 300, size=B)]
        for window in (-1, 5, 100):
            w = _tree_workload(rng, trees, prefixes, 8, 2, d, page, window, dtype)
            ref_o, ref_lse = oracle_full(w)
            tensors = device_inputs(w)
            for tile in (1, 2):
                o, lse, _ = run(pk, w, tensors, tile=tile)
                assert_close(o, lse, ref_o, ref_lse, dtype,
                             f"tree d={d} {dtype} P={page} trees={trees} prefixes={prefixes} "
                             f"w={window} tile={tile}")


def test_arbitrary_masks_and_empty_rows(pk):
    """Random (non-tree) bit patterns, masked prefixes, rows with no key at all
    (o = 0, lse = -inf), and requests without query rows."""
    rng = np.random.default_rng(71)
    mats = []
    for (q, L, density) in ((5, 70, 0.7), (3, 200, 0.3), (0, 40, 0.5), (9, 129, 0.9), (2, 64, 0.0)):
        m = rng.random((q, L)) < density
        if q > 2:
            m[1] = False          # one row sees nothing
        mats.append(m)
    for tile in (1, 2):
        for chunks in (0, 3):
            w = _tree_workload(rng, None, None, 4, 2, 128, 16, -1, W.BF16, mats=mats)
            ref_o, ref_lse = oracle_full(w)
            o, lse, _ = run(pk, w, tile=tile, num_kv_chunks=chunks)
            assert_close(o, lse, ref_o, ref_lse, w.dtype, f"arbitrary tile={tile} chunks={chunks}")


@pytest.mark.parametrize("batch", [4, 16, 64])
def test_tree_verify_full_size(pk, batch):
    w = W.tree_verify(batch=batch, poison=True)
    o, lse, p = run(pk, w)
    assert p.info["tile_rows"] == 32
    check_full(w, o, lse, f"tree verify b{batch}")


def test_chain_tree_equals_causal_verify(pk):
    w = W.config4(batch=16, num_kv_heads=8, poison=True)
    o_c, l_c, _ = run(pk, w)
    mats = [W.tree_topology_mask(int(kl) - int(ql), np.arange(int(ql)) - 1)
            for ql, kl in zip(w.qo_lens, w.kv_lens)]
    wt = W.Workload(**{**w.__dict__, "causal": False})
    wt.custom_mask, wt.mask_indptr = W.pack_custom_mask(mats)
    o_t, l_t, _ = run(pk, wt)
    assert np.abs(o_t - o_c).max() <= 1e-2
    assert np.abs(l_t - l_c).max() <= 1e-3
