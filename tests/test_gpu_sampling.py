"""Chain speculative sampling on the GPU against the oracle: accepted counts
and accepted tokens bit-exact (the accept test is one float32 product and
compare on both sides); drawn tokens equal to the oracle's, or -- where the
kernel's float32 running sums put s * total within their rounding error of a
boundary -- a draw that is valid within that error bound, checked in
float64; edge cases of the rule."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _run(pk, inp):
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    out, acc = pk.chain_speculative_sampling(t["draft_probs"], t["draft_token_ids"],
                                             t["target_probs"], t["accept_u"], t["sample_u"])
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64), acc.cpu().numpy().astype(np.int64)


def _fp32_sum_bound(V):
    """Relative error bound of the kernel's float32 running sums: an entry
    passes through at most log2(64) shuffle additions, 16 wave additions, one
    addition per earlier 1024-entry tile and the in-tile scan's log2(64) + 16."""
    return (6 + 16 + (V + 1023) // 1024 + 6 + 16 + 2) * 2.0 ** -24


def _valid_draw(w, s, k, rel=None):
    rel = _fp32_sum_bound(len(w)) if rel is None else rel
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    total = c[-1]
    thr = float(np.float32(s)) * total
    tol = rel * max(total, 1e-30)
    if not (0 <= k < len(w)) or w[k] <= 0:
        return False
    lo = c[k - 1] if k > 0 else 0.0
    if lo <= thr + tol and c[k] >= thr - tol:
        return True
    pos = np.nonzero(w > 0)[0]
    return k == pos[-1] and thr >= total - tol


def _check(pk, inp, what, max_boundary=None):
    got, got_acc = _run(pk, inp)
    want, want_acc = oracle.chain_speculative_sampling(**inp)
    assert np.array_equal(got_acc, want_acc), f"{what}: accepted counts differ"
    n = inp["draft_token_ids"].shape[1]
    boundary = 0
    for b in range(len(got_acc)):
        a = int(want_acc[b])
        assert np.array_equal(got[b, :a], want[b, :a]), f"{what}: accepted tokens b={b}"
        assert (got[b, a + 1:] == -1).all(), f"{what}: padding b={b}"
        if got[b, a] == want[b, a]:
            continue
        p = inp["target_probs"][b, a].astype(np.float32)
        w = np.maximum(p - inp["draft_probs"][b, a], 0) if a < n else p
        if a < n and w.sum() == 0:
            w = p
        assert _valid_draw(w, inp["sample_u"][b], int(got[b, a])), \
            f"{what}: b={b} drew {got[b, a]}, oracle {want[b, a]}"
        boundary += 1
    if max_boundary is not None:
        assert boundary <= max_boundary, f"{what}: {boundary} draws differ from the oracle"
    print(f"{what}: {boundary} of {len(got_acc)} draws within rounding of a boundary")
    return got, got_acc


# vocabularies that are multiples of 4 take the 16-byte-load path of the tile
# sums (4 and 1028: the smallest row, and a last tile of one load), the others
# the 4-byte path
@pytest.mark.parametrize("batch,n,vocab", [(16, 4, 5000), (8, 1, 1025), (5, 6, 1024),
                                           (3, 2, 7), (4, 3, 1), (6, 0, 3000), (2, 2, 4),
                                           (3, 1, 1028)])
def test_sampling_matches_oracle(pk, batch, n, vocab):
    inp = W.spec_sampling_inputs(variant=vocab + n, batch=batch, num_spec=n, vocab=vocab)
    _check(pk, inp, f"B={batch} n={n} V={vocab}")


def test_sampling_full_size(pk):
    # 64 requests x 4 drafts over a 128256-entry vocabulary
    inp = W.spec_sampling_inputs()
    got, acc = _check(pk, inp, "B=64 n=4 V=128256")
    assert 0 < acc.mean() < 4   # a correlated draft: some accepted, some rejected


def test_sampling_special_cases(pk):
    base = W.spec_sampling_inputs(variant=9, batch=12, num_spec=3, vocab=2000)
    # identical draft and target: every draft accepted, a bonus token drawn
    same = dict(base)
    same["draft_probs"] = np.ascontiguousarray(base["target_probs"][:, :3])
    _, acc = _check(pk, same, "identical")
    assert (acc == 3).all()
    # the target puts no mass on drafted tokens: rejected at once, drawn from p
    dis = {k: v.copy() for k, v in base.items()}
    for b in range(12):
        for t in range(3):
            dis["target_probs"][b, t, dis["draft_token_ids"][b, t]] = 0.0
    _, acc = _check(pk, dis, "no target mass on drafts")
    assert (acc == 0).all()
    # target = draft / 2 (unnormalised): residual all zero, the draw falls back to p
    half = {k: v.copy() for k, v in base.items()}
    half["target_probs"][:, :3] = half["draft_probs"] * np.float32(0.5)
    half["accept_u"][:] = np.float32(0.75)
    _, acc = _check(pk, half, "zero residual")
    assert (acc == 0).all()
    # ids outside the vocabulary are rejected, never read
    bad = {k: v.copy() for k, v in base.items()}
    bad["draft_token_ids"][:, 0] = np.where(np.arange(12) % 2 == 0, -1, 2000).astype(np.int32)
    got, acc = _run(pk, bad)
    assert (acc == 0).all() and (got[:, 1:] == -1).all()
    # uniforms at the top of [0, 1)
    top = {k: v.copy() for k, v in base.items()}
    top["sample_u"][:] = np.float32(0.99999994)
    _check(pk, top, "u near 1")
