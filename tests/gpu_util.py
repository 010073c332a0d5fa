"""Helpers for GPU tests: move seeded workloads to the device, run the library,
compare every output element against the oracle with the stated tolerances."""
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


def assert_close(o, lse, ref_o, ref_lse, dtype, what=""):
    assert o.shape == ref_o.shape and lse.shape == ref_lse.shape, f"{what}: shapes differ"
    if o.size == 0:   # a batch without query rows has nothing more to compare
        return
    do = np.abs(o.astype(np.float64) - ref_o)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    assert do.max() <= O_TOL[dtype], f"{what}: max |do| = {do.max():.3g} > {O_TOL[dtype]}"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf pattern of lse differs"
    if fin.any():
        dl = np.abs(lse[fin].astype(np.float64) - ref_lse[fin])
        assert dl.max() <= LSE_TOL, f"{what}: max |dlse| = {dl.max():.3g} > {LSE_TOL}"


def check_full(w, o, lse, what, ref=None, **kw):
    """Every output element of the workload against the float64 oracle.
    Returns the oracle's (o, lse) for reuse."""
    ref_o, ref_lse = ref if ref is not None else oracle_full(w, **kw)
    assert o.shape == ref_o.shape and lse.shape == ref_lse.shape, what
    assert_close(o, lse, ref_o, ref_lse, w.dtype, what)
    return ref_o, ref_lse
