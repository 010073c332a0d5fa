"""Repeated runs and replays of captured HIP graphs give the eager results bit
for bit: attention with and without the split merge, and chain speculative
sampling.  Each graph is replayed several times; before each replay its output
buffers are overwritten eagerly and other eager launches of the same plan (same
workspaces) run, with synchronisations between, so a replay that skips work,
repeats it or depends on state an eager call left behind does not pass."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import device_inputs, plan_for, require_gpu

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _bits(t):
    """An integer view of a tensor, so that equality is bitwise (and -inf
    compares equal to itself)."""
    return t.view({2: torch.int16, 4: torch.int32}[t.element_size()])


def _same(a, b):
    return a.shape == b.shape and torch.equal(_bits(a), _bits(b))


CASES = {
    # paged batch prefill, B 8 (one pass, no merge)
    "paged_b8": (lambda: W.config2(poison=False), {}),
    # paged batch prefill with the 127-key window
    "paged_b8_w127": (lambda: W.config2(window_left=127, poison=False), {}),
    # B 2, q 64, kv 65536 in 8 chunks: split tiles and the merge launch
    "split_q64": (lambda: W.config5(qo_len=64, poison=False),
                  {"num_kv_chunks": W.CONFIG5_CHUNKS}),
    # verify B 16, 4 queries per request, Hkv 8: the short-query kernel
    "verify_b16": (lambda: W.config4(batch=16, num_kv_heads=8, poison=False), {}),
    # verify B 64, Hkv 4: 624 tasks on 256 CUs, the later ones taken in start
    # order from the plan's task counter (which each launch leaves at zero)
    "verify_b64": (lambda: W.config4(batch=64, num_kv_heads=4, poison=False), {}),
}


@pytest.mark.parametrize("case", list(CASES))
def test_attention_graph_replays_equal_eager(pk, case):
    make, opts = CASES[case]
    w = make()
    q, k, v = device_inputs(w)
    p = plan_for(pk, w, **opts)
    if case == "split_q64":
        assert p.info["num_merge_items"] > 0
    o_ref, lse_ref = p.run(q, k, v)
    o_rep, lse_rep = p.run(q, k, v)
    torch.cuda.synchronize()
    assert torch.isfinite(o_ref.float()).all()
    # no order-dependent sums (the start-order task counter only picks which
    # work group computes a task): a second eager run is bit-identical
    assert _same(o_ref, o_rep) and _same(lse_ref, lse_rep), f"{case}: eager runs differ"

    o = torch.empty_like(o_ref)
    lse = torch.empty_like(lse_ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p.run(q, k, v, out=o, lse=lse)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        o_rep, lse_rep = p.run(q, k, v)          # eager work on the same workspaces
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(o, o_ref) and _same(lse, lse_ref), f"{case}: replay {i} differs"
        assert _same(o_rep, o_ref), f"{case}: eager run {i} between replays differs"
    del g


def test_graph_with_two_plans_and_rotating_pools(pk):
    """One graph holding runs of two plans over two copies of the K/V pools (the
    benchmark's timing pattern): each output equals its eager run."""
    w = W.config4(batch=16, num_kv_heads=8, poison=False)
    w2 = W.config2(window_left=127, poison=False)
    (qa, ka, va), (qb, kb, vb) = device_inputs(w), device_inputs(w2)
    pa, pb = plan_for(pk, w), plan_for(pk, w2)
    ka2, va2, kb2, vb2 = ka.clone(), va.clone(), kb.clone(), vb.clone()
    ref = [pa.run(qa, ka, va), pb.run(qb, kb, vb)]
    torch.cuda.synchronize()
    outs = [(torch.empty_like(r[0]), torch.empty_like(r[1])) for r in ref * 2]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.run(qa, ka, va, out=outs[0][0], lse=outs[0][1])
        pb.run(qb, kb, vb, out=outs[1][0], lse=outs[1][1])
        pa.run(qa, ka2, va2, out=outs[2][0], lse=outs[2][1])
        pb.run(qb, kb2, vb2, out=outs[3][0], lse=outs[3][1])
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o, lse in outs:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, lse) in enumerate(outs):
            r = ref[j % 2]
            assert _same(o, r[0]) and _same(lse, r[1]), f"replay {i}, run {j} differs"
    del g


def test_sampling_graph_replays_equal_eager(pk):
    inp = W.spec_sampling_inputs(batch=16, vocab=50000)
    t = {k: torch.from_numpy(np.ascontiguousarray(x)).cuda() for k, x in inp.items()}
    args = (t["draft_probs"], t["draft_token_ids"], t["target_probs"], t["accept_u"],
            t["sample_u"])
    B = inp["draft_token_ids"].shape[0]
    V = inp["target_probs"].shape[2]
    ws = torch.empty(pk.load_library().pkv_chain_speculative_sampling_workspace_size(B, V),
                     dtype=torch.uint8, device="cuda")
    out_ref, acc_ref = pk.chain_speculative_sampling(*args, workspace=ws)
    out2, acc2 = pk.chain_speculative_sampling(*args, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_ref, out2) and torch.equal(acc_ref, acc2)
    out = torch.empty_like(out_ref)
    acc = torch.empty_like(acc_ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pk.chain_speculative_sampling(*args, out=out, num_accepted=acc, workspace=ws)
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        out.fill_(-7)
        acc.fill_(-7)
        pk.chain_speculative_sampling(*args, workspace=ws)   # eager use of the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref) and torch.equal(acc, acc_ref), f"replay {i} differs"
    del g
