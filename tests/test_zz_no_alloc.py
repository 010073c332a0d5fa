"""The allocation-free speculative-sampling entry point against the one that
takes a caller workspace: same inputs, bit-identical accepted counts and
tokens, on two calls in a row (the second smaller, so the library's shared
per-GPU array holds the first call's larger contents), and when captured in a
HIP graph and replayed."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _inputs(batch, num_spec, vocab, variant):
    inp = W.spec_sampling_inputs(variant=variant, batch=batch, num_spec=num_spec, vocab=vocab)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    return (t["draft_probs"], t["draft_token_ids"], t["target_probs"], t["accept_u"],
            t["sample_u"])


def _both(pk, args):
    B, n = args[1].shape
    ref_out, ref_acc = pk.chain_speculative_sampling(*args)
    out = torch.full((B, n + 1), -7, dtype=torch.int32, device="cuda")
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    pk.chain_speculative_sampling_no_alloc(*args, out=out, num_accepted=acc)
    torch.cuda.synchronize()
    return ref_out, ref_acc, out, acc


def test_no_alloc_equals_workspace_entry_point(pk):
    # the benchmark's size first, then a smaller batch and vocabulary (and a
    # vocabulary not a multiple of 4, which takes the 4-byte load path)
    for batch, n, vocab, variant in ((64, 4, 128256, 0), (5, 3, 3001, 1)):
        args = _inputs(batch, n, vocab, variant)
        ref_out, ref_acc, out, acc = _both(pk, args)
        assert torch.equal(acc, ref_acc), (batch, vocab)
        assert torch.equal(out, ref_out), (batch, vocab)
        assert (acc >= 0).all() and (acc <= n).all()


def test_no_alloc_under_graph_capture(pk):
    args = _inputs(16, 4, 32000, 2)
    ref_out, ref_acc, _, _ = _both(pk, args)
    out = torch.full_like(ref_out, -7)
    acc = torch.full_like(ref_acc, -7)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pk.chain_speculative_sampling_no_alloc(*args, out=out, num_accepted=acc)
    for _ in range(3):
        out.fill_(-7)
        acc.fill_(-7)
        # another call on the shared array between replays (ordered on one stream)
        other = _inputs(3, 2, 5000, 3)
        pk.chain_speculative_sampling_no_alloc(
            *other, out=torch.empty((3, 3), dtype=torch.int32, device="cuda"),
            num_accepted=torch.empty(3, dtype=torch.int32, device="cuda"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(acc, ref_acc) and torch.equal(out, ref_out)
