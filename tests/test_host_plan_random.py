"""The scheduler on seeded random batches, on the CPU (no device call).

For each batch the plan's task list must tile the work exactly: every packed
(position, head-in-group) row of every (request, kv head) in one row tile, and
the chunks of each row tile disjoint and covering exactly the keys that row
sees under the bottom-right causal mask and the left window (PR #362, Summary;
PR #339, "Why window_size_right stays -1"), restricted to [kv_begin, kv_end).
Split tiles use consecutive partial slots, one merge item each.  The batches mix
empty requests, requests shorter than a page, GQA groups 1-8, page sizes 1-64,
both tile shapes, forced chunk counts and split sizes, custom masks and key
ranges.
"""
import numpy as np
import pytest

import paged_kv_cache_prefill_amd as pk
import workloads as W


def _random_case(rng):
    batch = int(rng.integers(1, 7))
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 3, 4, 6, 8]))
    head_dim = int(rng.choice([64, 128, 128, 256]))
    page = int(rng.choice([1, 2, 3, 5, 16, 16, 64]))
    mask = rng.random() < 0.15
    causal = (not mask) and rng.random() < 0.6
    qo = rng.integers(0, 71, size=batch)
    qo[rng.random(batch) < 0.15] = 0                       # empty requests
    extra = rng.integers(0, 301, size=batch)
    kv = qo + extra if causal else np.maximum(1, rng.integers(0, 371, size=batch))
    kv = np.where((qo == 0) & (rng.random(batch) < 0.3), 0, kv)   # no rows, no keys
    window = int(rng.choice([-1, -1, 0, 1, 7, 31, 64, 127, 1000]))
    w = W.build("random", qo, kv, hkv * group, hkv, head_dim, page, causal, window, "bf16",
                seed=int(rng.integers(1 << 30)), values=False)
    opts = {}
    if head_dim != 256:
        opts["tile"] = int(rng.choice([0, 0, 1, 2]))
    r = rng.random()
    if r < 0.2:
        opts["num_kv_chunks"] = int(rng.choice([1, 2, 3, 7]))
    elif r < 0.35:
        opts["split_tiles"] = int(rng.choice([1, 2, 5]))
    if rng.random() < 0.15:
        kb = int(rng.integers(0, 64))
        opts["kv_begin"] = kb
        opts["kv_end"] = int(rng.choice([-1, kb + int(rng.integers(1, 200))]))
    if mask:
        mats = [(rng.random((int(q), int(k))) < 0.5) for q, k in zip(qo, kv)]
        w.custom_mask, w.mask_indptr = W.pack_custom_mask(mats)
    return w, opts


def _visible(i, Q, L, causal, window):
    hi = i + L - Q if causal else L - 1
    lo = 0 if window == -1 else max(0, L + i - Q - window)
    return lo, min(hi, L - 1)


def _check(w, opts):
    p = pk.plan_host(**w.plan_args(), **opts)
    info = p.info
    items = p.work_items()
    G = w.num_qo_heads // w.num_kv_heads
    NK, TR = info["tile_keys"], info["tile_rows"]
    kb, ke = opts.get("kv_begin", 0), opts.get("kv_end", -1)
    tiles = {}
    for (b, kvh, row0, nrows, lo, end, slot, tb) in items:
        if nrows == 0:                       # padding record of an XCD-grouped list
            assert slot == -1
            continue
        # an empty key range is a task too: its rows see no key and are written (0, -inf)
        assert 0 < nrows <= TR and tb % NK == 0 and tb <= max(lo, 0)
        tiles.setdefault((b, kvh, row0, nrows), []).append((lo, end, slot))
    if any(r[3] == 0 for r in items):
        assert len(items) % 8 == 0
    split = [c for c in tiles.values() if len(c) > 1]
    assert len(split) == info["num_merge_items"]
    slots = sorted(s for c in tiles.values() for (_, _, s) in c if s >= 0)
    assert slots == list(range(info["num_partial_slots"]))
    for c in split:
        s = sorted(x[2] for x in c)
        assert s[0] >= 0 and s == list(range(s[0], s[0] + len(s)))
    for b in range(w.batch_size):
        Q, L = int(w.qo_lens[b]), int(w.kv_lens[b])
        for kvh in range(w.num_kv_heads):
            mine = sorted(t for t in tiles if t[0] == b and t[1] == kvh)
            rows = [r for (_, _, row0, nrows) in mine for r in range(row0, row0 + nrows)]
            for key in mine:
                chunks = sorted(tiles[key])
                live = [c for c in chunks if c[0] < c[1]]
                for (_, e0, _), (a1, _, _) in zip(live, live[1:]):
                    assert e0 <= a1, (b, kvh, key)       # disjoint
                _, _, row0, nrows = key
                for r in range(row0, row0 + nrows):
                    lo, hi = _visible(r // G, Q, L, w.causal, w.window_left)
                    lo, hi = max(lo, kb), min(hi, L - 1 if ke < 0 else ke - 1)
                    got = sum(max(0, min(e, hi + 1) - max(a, lo)) for (a, e, _) in chunks)
                    assert got == max(0, hi - lo + 1), (b, kvh, r, lo, hi, chunks)
            assert sorted(rows) == list(range(Q * G)), (b, kvh)   # each row in one tile
    return info


@pytest.mark.parametrize("block", range(16))
def test_random_batches_are_tiled_exactly(block):
    rng = np.random.default_rng(1000 + block)
    for case in range(100):
        w, opts = _random_case(rng)
        try:
            _check(w, opts)
        except AssertionError as e:
            raise AssertionError(f"block {block} case {case}: qo {w.qo_lens.tolist()} "
                                 f"kv {w.kv_lens.tolist()} Hq/Hkv {w.num_qo_heads}/"
                                 f"{w.num_kv_heads} D {w.head_dim} page {w.page_size} "
                                 f"causal {w.causal} window {w.window_left} "
                                 f"mask {w.custom_mask is not None} opts {opts}") from e
