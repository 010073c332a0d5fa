"""GPU parity on seeded random batches: every output element against the
float64 oracle, with the tolerances of the other parity tests (max |do| <= 1e-2
fp16 / 2e-2 bf16, |dlse| <= 1e-3).

Each batch draws its own combination of what the grid tests vary one or two
at a time: dtype, head_dim 64/128/256, GQA group 1-8, page size 1-128,
bottom-right causal or not (PR #362, Summary), a left window (PR #339, "Why
window_size_right stays -1"), a topology mask (PR #362, Architecture / design
notes), a logits soft-cap, FP8 E4M3 caches, the tile shape, forced KV chunks
or split sizes, a key range, and NHD or HND pool strides; with empty requests,
requests shorter than a page and NaN in every unreferenced pool slot.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import assert_close, require_gpu, to_device, torch_dtype

pytestmark = pytest.mark.gpu

KS, VS = 0.5, 2.0   # FP8 k_scale / v_scale


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _case(rng):
    dtype = W.BF16 if rng.random() < 0.6 else W.FP16
    d = int(rng.choice([64, 128, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 3, 4, 6, 8]))
    page = int(rng.choice([1, 2, 3, 5, 16, 16, 64, 128]))
    mask = rng.random() < 0.2
    causal = (not mask) and rng.random() < 0.6
    batch = int(rng.integers(1, 6))
    qo = rng.integers(0, 90, size=batch)
    qo[rng.random(batch) < 0.15] = 0
    kv = qo + rng.integers(0, 400, size=batch) if causal else \
        np.maximum(1, rng.integers(0, 500, size=batch))
    kv = np.where((qo == 0) & (rng.random(batch) < 0.3), 0, kv)
    window = int(rng.choice([-1, -1, 0, 1, 7, 31, 64, 127, 1000]))
    w = W.build("random", qo, kv, hkv * group, hkv, d, page, causal, window, dtype,
                seed=int(rng.integers(1 << 30)), poison=True)
    if mask:
        mats = [(rng.random((int(q), int(k))) < 0.6) for q, k in zip(qo, kv)]
        w.custom_mask, w.mask_indptr = W.pack_custom_mask(mats)
    w.logits_soft_cap = float(rng.choice([0.0, 0.0, 0.0, 5.0, 30.0]))
    fp8 = rng.random() < 0.25
    opts = {}
    if d != 256:
        opts["tile"] = int(rng.choice([0, 0, 1, 2]))
    r = rng.random()
    if r < 0.2:
        opts["num_kv_chunks"] = int(rng.choice([1, 2, 3, 7]))
    elif r < 0.3:
        opts["split_tiles"] = int(rng.choice([1, 2]))
    if rng.random() < 0.1:
        kb = int(rng.integers(0, 64))
        opts["kv_begin"] = kb
        opts["kv_end"] = int(rng.choice([-1, kb + int(rng.integers(1, 300))]))
    hnd = rng.random() < 0.3
    return w, fp8, hnd, opts


def _describe(w, fp8, hnd, opts):
    return (f"qo {w.qo_lens.tolist()} kv {w.kv_lens.tolist()} {w.dtype} D {w.head_dim} "
            f"Hq/Hkv {w.num_qo_heads}/{w.num_kv_heads} page {w.page_size} causal {w.causal} "
            f"window {w.window_left} mask {w.custom_mask is not None} "
            f"cap {w.logits_soft_cap} fp8 {fp8} {'HND' if hnd else 'NHD'} opts {opts}")


def _pool(t, hnd):
    # HND: the same pool stored [pages, heads, page_size, dim], passed as a
    # strided [pages, page_size, heads, dim] view
    return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) if hnd else t


def _check_case(pk, rng, what):
    w, fp8, hnd, opts = _case(rng)
    what = f"{what}: {_describe(w, fp8, hnd, opts)}"
    qf, kf, vf = w.float_inputs()
    plan_opts = dict(opts)
    if fp8:
        kc, vc = W.e4m3_pools(w, int(rng.integers(1 << 30)), KS, VS)
        kf, vf = oracle.decode_e4m3(kc, KS), oracle.decode_e4m3(vc, VS)
        k, v = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
        plan_opts.update(kv_dtype="fp8_e4m3", k_scale=KS, v_scale=VS)
    else:
        k, v = to_device(w.k_pool, w.dtype), to_device(w.v_pool, w.dtype)
    a = w.plan_args()
    ref_args = {key: val for key, val in a.items() if key != "head_dim"}
    kr = {}
    if "kv_begin" in opts:
        kr = dict(kv_begin=opts["kv_begin"],
                  kv_end=None if opts["kv_end"] < 0 else opts["kv_end"])
    ref_o, ref_lse = oracle.attention(qf, kf, vf, **ref_args, **kr)
    q = to_device(w.q, w.dtype)
    print(what, flush=True)
    p = pk.plan(**a, dtype=torch_dtype(w.dtype), **plan_opts)
    o, lse = p.run(q, _pool(k, hnd), _pool(v, hnd))
    torch.cuda.synchronize()
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_lse, w.dtype, what)


@pytest.mark.parametrize("block", range(16))
def test_random_batches_match_the_oracle(pk, block):
    rng = np.random.default_rng(zlib.crc32(f"random-batches-{block}".encode()))
    for case in range(24):
        _check_case(pk, rng, f"block {block} case {case}")
