"""Plan validation on corrupted inputs, on the CPU (no device call).

A valid batch is corrupted in one field at a time (decreasing or offset
indptrs, last-page lengths out of range, negative or huge page ids, head
counts GQA cannot divide, unsupported head_dim or page size, windows below
-1, a non-positive or non-finite sm_scale, causal requests shorter than their
queries, inconsistent topology masks, key ranges, chunk and tile options,
soft-caps and FP8 scales).  Every call must either be refused with a
PkvError (PR #399, What changed: inputs the kernels would compute wrongly are
refused before any compute) or return a plan whose task list still tiles the
batch; the library must never crash or read outside the arrays it is given.
"""
import numpy as np
import pytest

import paged_kv_cache_prefill_amd as pk
import workloads as W


def _valid(rng):
    batch = int(rng.integers(1, 5))
    qo = rng.integers(1, 40, size=batch)
    kv = qo + rng.integers(0, 100, size=batch)
    w = W.build("fuzz", qo, kv, 8, 2, 128, int(rng.choice([1, 3, 16])), True, -1, "bf16",
                seed=int(rng.integers(1 << 30)), values=False)
    args = {k: (np.array(v, copy=True) if isinstance(v, np.ndarray) else v)
            for k, v in w.plan_args().items()}
    return w, args, {}


def _corrupt(rng, w, args, opts):
    """One random corruption of a valid plan call; returns its name."""
    B = w.batch_size
    kinds = ["qo_dec", "qo_first", "qo_huge", "kv_dec", "kv_first", "kv_len", "last0",
             "last_big", "last_neg", "page_neg", "page_huge", "heads", "kv_heads0", "head_dim",
             "page0", "page_neg_size", "window", "scale0", "scale_neg", "scale_nan",
             "scale_inf", "causal_short", "mask_causal", "mask_dec", "mask_short",
             "kv_range", "kv_begin_neg", "chunks_neg", "split_neg", "tile_bad", "cap_neg",
             "cap_nan", "fp8_scale_neg", "fp8_scale_nan", "indices_short", "rows_huge"]
    kind = str(rng.choice(kinds))
    i = int(rng.integers(0, B))
    if kind == "qo_dec" and B > 1:
        args["qo_indptr"][i + 1] = args["qo_indptr"][i] - 1
    elif kind == "qo_first":
        args["qo_indptr"][0] = 1
    elif kind == "qo_huge":
        args["qo_indptr"][-1] = 2**31 - 1
    elif kind == "kv_dec" and B > 1:
        args["kv_indptr"][i + 1] = args["kv_indptr"][i] - 1
    elif kind == "kv_first":
        args["kv_indptr"][0] = 1
    elif kind == "kv_len":
        args["kv_indptr"][-1] += int(rng.choice([-1, 1, 1000]))
    elif kind == "last0":
        args["kv_last_page_len"][i] = 0
    elif kind == "last_big":
        args["kv_last_page_len"][i] = args["page_size"] + 1
    elif kind == "last_neg":
        args["kv_last_page_len"][i] = -5
    elif kind == "page_neg":
        args["kv_page_indices"][int(rng.integers(0, len(args["kv_page_indices"])))] = -1
    elif kind == "page_huge":
        args["kv_page_indices"][int(rng.integers(0, len(args["kv_page_indices"])))] = 2**31 - 1
    elif kind == "heads":
        args["num_qo_heads"] = 7
    elif kind == "kv_heads0":
        args["num_kv_heads"] = 0
    elif kind == "head_dim":
        args["head_dim"] = int(rng.choice([0, 32, 96, 512, -64]))
    elif kind == "page0":
        args["page_size"] = 0
    elif kind == "page_neg_size":
        args["page_size"] = -16
    elif kind == "window":
        args["window_left"] = int(rng.choice([-2, -1000]))
    elif kind == "scale0":
        args["sm_scale"] = 0.0
    elif kind == "scale_neg":
        args["sm_scale"] = -0.1
    elif kind == "scale_nan":
        args["sm_scale"] = float("nan")
    elif kind == "scale_inf":
        args["sm_scale"] = float("inf")
    elif kind == "causal_short":
        # more query rows than keys under the causal mask
        args["qo_indptr"][1:] = args["qo_indptr"][1:] + 10_000
    elif kind == "mask_causal":
        mats = [np.ones((int(q), int(k)), bool) for q, k in zip(w.qo_lens, w.kv_lens)]
        opts["custom_mask"], opts["mask_indptr"] = W.pack_custom_mask(mats)   # causal stays 1
    elif kind in ("mask_dec", "mask_short"):
        args["causal"] = False
        mats = [np.ones((int(q), int(k)), bool) for q, k in zip(w.qo_lens, w.kv_lens)]
        data, ind = W.pack_custom_mask(mats)
        ind = ind.copy()
        if kind == "mask_dec" and B > 1:
            ind[i + 1] = ind[i] - 1
        else:
            ind[i + 1] -= 1
        opts["custom_mask"], opts["mask_indptr"] = data, ind
    elif kind == "kv_range":
        opts["kv_begin"], opts["kv_end"] = 50, 10
    elif kind == "kv_begin_neg":
        opts["kv_begin"] = -3
    elif kind == "chunks_neg":
        opts["num_kv_chunks"] = -1
    elif kind == "split_neg":
        opts["split_tiles"] = -2
    elif kind == "tile_bad":
        opts["tile"] = int(rng.choice([3, -1]))
    elif kind == "cap_neg":
        opts["logits_soft_cap"] = -1.0
    elif kind == "cap_nan":
        opts["logits_soft_cap"] = float("nan")
    elif kind == "fp8_scale_neg":
        opts.update(kv_dtype="fp8_e4m3", k_scale=-1.0)
    elif kind == "fp8_scale_nan":
        opts.update(kv_dtype="fp8_e4m3", v_scale=float("nan"))
    elif kind == "indices_short":
        args["kv_page_indices"] = args["kv_page_indices"][:-1]
    elif kind == "rows_huge":
        # without the causal bound: 2^29 query rows x 4 heads per group would
        # overflow the kernels' 32-bit packed-row arithmetic
        args["causal"] = False
        args["qo_indptr"][1:] = args["qo_indptr"][1:] + (1 << 29)
    return kind


@pytest.mark.parametrize("block", range(6))
def test_corrupted_plans_are_refused_or_valid(block):
    rng = np.random.default_rng(7000 + block)
    refused = 0
    for case in range(100):
        w, args, opts = _valid(rng)
        kind = _corrupt(rng, w, args, opts)
        try:
            p = pk.plan_host(**args, **opts)
        except pk.PkvError as e:
            refused += 1
            assert str(e), kind
            continue
        # accepted: the corruption left a valid call; its plan must still be consistent
        items = p.work_items()
        info = p.info
        assert info["total_q_rows"] == int(np.asarray(args["qo_indptr"])[-1]), kind
        assert len(items) == info["num_work_items"], kind
        slots = sorted(int(s) for s in items[:, 6] if s >= 0)
        assert slots == list(range(info["num_partial_slots"])), kind
    assert refused >= 50   # most corruptions are refusals
