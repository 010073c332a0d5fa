"""FP8 E4M3 K/V caches on the GPU against the oracle (values = code x scale,
decoded by the oracle from the format's definition): every head dim, page
address path and tile shape, windows, split chunks, NaN-poisoned unreferenced
codes, custom topology masks and logits soft-caps alone and together, and
full-size verify and prefill compared on every output element."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import O_TOL, LSE_TOL, assert_close, require_gpu, to_device, torch_dtype

pytestmark = pytest.mark.gpu

KS, VS = 0.5, 2.0


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _run(pk, w, kc, vc, **opts):
    q = to_device(w.q, w.dtype)
    k = torch.from_numpy(kc).cuda()
    v = torch.from_numpy(vc).cuda()
    p = pk.plan(**w.plan_args(), dtype=torch_dtype(w.dtype), kv_dtype="fp8_e4m3", k_scale=KS,
                v_scale=VS, **opts)
    o, lse = p.run(q, k, v)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), p


def _floats(w, kc, vc):
    q, _, _ = w.float_inputs()
    return q, oracle.decode_e4m3(kc, KS), oracle.decode_e4m3(vc, VS)


def _oracle(w, kc, vc):
    q, k, v = _floats(w, kc, vc)
    a = w.plan_args()
    del a["head_dim"]
    return oracle.attention(q, k, v, **a)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("page", [1, 3, 8, 16, 256])
def test_fp8_tiny(pk, d, page):
    # pages 1 and 3 take the per-lane page-table path; power-of-two pages
    # that hold a whole load instruction's rows (>= 64 / (d / 16) keys: 16,
    # 8, 4 for d = 64, 128, 256) take the scalar page-id path, 256 with
    # tiles that start inside a page
    rng = np.random.default_rng(d * 10 + page)
    qo = [1, 23, 70]
    kv = [40, 23, 190]
    for causal, wl in ((True, -1), (False, 12), (True, 60)):
        w = W.build("fp8", qo, kv, 8, 2, d, page, causal, wl, W.BF16,
                    seed=int(rng.integers(1 << 30)))
        kc, vc = W.e4m3_pools(w, int(rng.integers(1 << 30)), KS, VS)
        ref_o, ref_lse = _oracle(w, kc, vc)
        for tile in ((1,) if d == 256 else (1, 2)):
            for chunks in (0, 3):
                o, lse, _ = _run(pk, w, kc, vc, tile=tile, num_kv_chunks=chunks)
                assert_close(o, lse, ref_o, ref_lse, w.dtype,
                             f"fp8 d={d} P={page} causal={causal} w={wl} tile={tile} "
                             f"chunks={chunks}")


def test_fp8_fp16_queries(pk):
    w = W.build("fp8h", [17, 5], [90, 300], 8, 4, 128, 16, True, -1, W.FP16, seed=5)
    kc, vc = W.e4m3_pools(w, 6, KS, VS)
    ref_o, ref_lse = _oracle(w, kc, vc)
    o, lse, _ = _run(pk, w, kc, vc)
    assert_close(o, lse, ref_o, ref_lse, w.dtype, "fp8 with fp16 q")


@pytest.mark.parametrize("case", ["verify_b64", "prefill_b8"])
def test_fp8_full_size(pk, case):
    w = W.config4(batch=64, num_kv_heads=8, values=True) if case == "verify_b64" else \
        W.config2(values=True)
    kc, vc = W.e4m3_pools(w, 77, KS, VS, poison=True)
    o, lse, _ = _run(pk, w, kc, vc)
    ref_o, ref_lse = _oracle(w, kc, vc)   # every output element
    assert_close(o, lse, ref_o, ref_lse, w.dtype, f"fp8 {case}")


def _tree_fp8(rng, d, page, window, cap, batch):
    prefixes = [int(x) for x in rng.integers(0, 300, size=batch)]
    mats = [W.tree_topology_mask(p, W.random_tree_parents(rng, int(n)))
            for p, n in zip(prefixes, rng.integers(1, 12, size=batch))]
    w = W.build("fp8tree", [m.shape[0] for m in mats], [m.shape[1] for m in mats], 8, 2, d,
                page, False, window, W.BF16, seed=int(rng.integers(1 << 30)))
    w.custom_mask, w.mask_indptr = W.pack_custom_mask(mats)
    w.logits_soft_cap = cap
    return w


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("page", [1, 3, 16])
@pytest.mark.parametrize("mask,cap", [(True, 0.0), (False, 1.5), (True, 2.0)])
def test_fp8_mask_and_soft_cap(pk, d, page, mask, cap):
    """Topology masks and soft-caps over E4M3 caches: the cap acts on the
    decoded logit sm_scale * q . (code * k_scale), so a cap of 1.5 or 2 with
    N(0, 1)-like logits bends most of them; every page path and tile shape."""
    rng = np.random.default_rng(zlib.crc32(repr((d, page, mask, cap)).encode()))
    for window in (-1, 7, 150):
        if mask:
            w = _tree_fp8(rng, d, page, window, cap, int(rng.integers(1, 5)))
        else:
            w = W.build("fp8cap", [1, 23, 70, 130], [40, 23, 190, 400], 8, 2, d, page, True,
                        window, W.BF16, seed=int(rng.integers(1 << 30)))
            w.logits_soft_cap = cap
        kc, vc = W.e4m3_pools(w, int(rng.integers(1 << 30)), KS, VS)
        ref_o, ref_lse = _oracle(w, kc, vc)
        for tile in ((1,) if d == 256 else (1, 2)):
            for chunks in (0, 3):
                o, lse, _ = _run(pk, w, kc, vc, tile=tile, num_kv_chunks=chunks)
                assert_close(o, lse, ref_o, ref_lse, w.dtype,
                             f"fp8 d={d} P={page} mask={mask} cap={cap} w={window} "
                             f"tile={tile} chunks={chunks}")


@pytest.mark.parametrize("cap", [0.0, 30.0])
def test_fp8_tree_verify_full_size(pk, cap):
    """The tree-verify workload (B16, Hkv 8, 8-node trees after 512..8192-key
    prefixes) over E4M3 caches, with and without a soft-cap, every element."""
    w = W.tree_verify(batch=16, values=True)
    w.logits_soft_cap = cap
    kc, vc = W.e4m3_pools(w, 91, KS, VS, poison=True)
    o, lse, p = _run(pk, w, kc, vc)
    assert p.info["tile_rows"] == 32
    ref_o, ref_lse = _oracle(w, kc, vc)
    assert_close(o, lse, ref_o, ref_lse, w.dtype, f"fp8 tree verify cap={cap}")


def test_fp8_refusals(pk):
    w = W.build("fp8r", [3], [20], 4, 2, 64, 16, True, -1, W.BF16, seed=9)
    p = pk.plan(**w.plan_args(), dtype=torch.bfloat16, kv_dtype="fp8_e4m3")
    q = to_device(w.q, w.dtype)
    kb = to_device(w.k_pool, w.dtype)
    with pytest.raises(pk.PkvError, match="dtype"):
        p.run(q, kb, kb)


@pytest.mark.parametrize("dtype", [W.BF16, W.FP16])
@pytest.mark.parametrize("d,tile", [(64, 1), (64, 2), (128, 1), (128, 2), (256, 1)])
def test_fp8_every_code_decodes_exactly(pk, dtype, d, tile):
    """One visible key per request makes each output row that key's V row times
    v_scale, exactly (the softmax weight is 1): every finite E4M3 code at every
    byte position of a 16-byte load then comes out bit-exact in the query dtype,
    on the prefill and on the short-query tile."""
    B = 4096 // d                      # B * d / 16 = 256 (load, position) slots per byte lane
    rng = np.random.default_rng(d * 7 + tile)
    pages = rng.permutation(B).astype(np.int32)
    n = np.arange(B)[:, None] * (d // 16) + np.arange(d)[None, :] // 16
    codes = ((n + np.arange(d)[None, :] % 16) % 256).astype(np.uint8)   # [request, dim]
    codes[(codes & 0x7F) == 0x7F] = 0                                   # the two NaN codes
    vc = np.zeros((B, 1, 1, d), np.uint8)
    vc[pages, 0, 0, :] = codes
    kc = W.e4m3_codes(rng.standard_normal((B, 1, 1, d), dtype=np.float32))
    ar = np.arange(B + 1, dtype=np.int32)
    p = pk.plan(ar, ar, pages, np.ones(B, np.int32), 4, 1, d, 1, True, dtype=torch_dtype(dtype),
                kv_dtype="fp8_e4m3", k_scale=KS, v_scale=VS, tile=tile)
    q = torch.randn((B, 4, d), dtype=torch.float32).to(torch_dtype(dtype)).cuda()
    o, lse = p.run(q, torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda())
    torch.cuda.synchronize()
    assert p.info["tile_rows"] in ((128, 64) if tile == 1 else (16, 32))   # the tile asked for
    want = oracle.decode_e4m3(codes, VS)                                # exact in fp16 and bf16
    got = o.double().cpu().numpy()
    for h in range(4):
        bad = np.nonzero(got[:, h, :] != want)
        assert bad[0].size == 0, (f"head {h}: {bad[0].size} codes differ, first request "
                                  f"{bad[0][0]} dim {bad[1][0]} code {codes[bad][0]:#04x}")
    assert np.isfinite(lse.cpu().numpy()).all()
