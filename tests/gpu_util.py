"""Helpers for GPU tests: move seeded workloads to the device, run the library,
compare against the oracle with the stated tolerances."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

# max |o - o_ref| and |lse - lse_ref| allowed against the float64 oracle
O_TOL = {W.FP16: 1e-2, W.BF16: 2e-2}
LSE_TOL = 1e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import paged_kv_cache_prefill_amd as pk
    pk.load_library()  # raises if the HIP library is missing: no fallback
    return pk


def to_device(arr, dtype, device="cuda"):
    if dtype == W.BF16:
        return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == W.BF16 else torch.float16


def device_inputs(w, device="cuda"):
    return (to_device(w.q, w.dtype, device), to_device(w.k_pool, w.dtype, device),
            to_device(w.v_pool, w.dtype, device))


def plan_for(pk, w, **opts):
    a = w.plan_args()
    return pk.plan(**a, dtype=torch_dtype(w.dtype), **opts)


def run(pk, w, tensors=None, **opts):
    q, k, v = tensors if tensors is not None else device_inputs(w)
    p = plan_for(pk, w, **opts)
    o, lse = p.run(q, k, v)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), p


def oracle_full(w, **kw):
    q, k, v = w.float_inputs()
    a = w.plan_args()
    del a["head_dim"]
    return oracle.attention(q, k, v, **a, **kw)


def oracle_rows(w, b, rows, heads, floats=None, **kw):
    q, k, v = floats if floats is not None else w.float_inputs()
    a = w.plan_args()
    del a["head_dim"]
    return oracle.attention_rows(q, k, v, **a, b=b, rows=rows, heads=heads, **kw)


def assert_close(o, lse, ref_o, ref_lse, dtype, what=""):
    do = np.abs(o.astype(np.float64) - ref_o)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    assert do.max() <= O_TOL[dtype], f"{what}: max |do| = {do.max():.3g} > {O_TOL[dtype]}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf pattern of lse differs"
    if fin.any():
        dl = np.abs(lse[fin].astype(np.float64) - ref_lse[fin])
        assert dl.max() <= LSE_TOL, f"{what}: max |dlse| = {dl.max():.3g} > {LSE_TOL}"


def sample_rows(rng, w, per_request=3, heads=4):
    """(b, rows, heads) samples, always including the first and last row."""
    out = []
    for b in range(w.batch_size):
        ql = int(w.qo_lens[b])
        if ql == 0:
            continue
        rows = sorted({0, ql - 1, *rng.integers(0, ql, size=per_request).tolist()})
        hs = sorted({0, w.num_qo_heads - 1,
                     *rng.integers(0, w.num_qo_heads, size=heads).tolist()})
        out.append((b, rows, hs))
    return out


def check_sampled(w, o, lse, rng, what, floats=None, per_request=3, heads=4, **kw):
    floats = floats if floats is not None else w.float_inputs()
    for b, rows, hs in sample_rows(rng, w, per_request, heads):
        ref_o, ref_lse = oracle_rows(w, b, rows, hs, floats=floats, **kw)
        base = int(w.qo_indptr[b])
        go = o[np.ix_([base + r for r in rows], hs)]
        gl = lse[np.ix_([base + r for r in rows], hs)]
        assert_close(go, gl, ref_o, ref_lse, w.dtype, f"{what} b={b}")
