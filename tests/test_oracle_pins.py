"""Pins for the CPU oracle: it is checked against things other than itself.

* hand-derived golden fixtures (tests/golden/),
* a literal per-element brute force on a grid of tiny inputs,
* closed forms (K = 0 gives lse = log(#visible keys); V = 1 gives o = 1),
* library routines (torch scaled_dot_product_attention / logsumexp on CPU),
* invariants (wide window == no window, GQA == replicated heads, page
  relabelling, last verify row == decode, split + merge == unsplit),
* non-vacuity (windowed / causal / GQA variants really differ),
* planted mistakes: each pin function rejects a deliberately wrong oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers building small random paged problems (float64 values, no rounding)
# ---------------------------------------------------------------------------

def small_problem(rng, qo_lens, kv_lens, hq, hkv, d, page_size, permute=True):
    kv_indptr, ids, last, num_pages = workloads.make_page_table(
        rng, kv_lens, page_size, pool_factor=1.5, permute=permute)
    qo_indptr = np.zeros(len(qo_lens) + 1, dtype=np.int64)
    qo_indptr[1:] = np.cumsum(qo_lens)
    q = rng.standard_normal((int(qo_indptr[-1]), hq, d))
    k = rng.standard_normal((num_pages, page_size, hkv, d))
    v = rng.standard_normal((num_pages, page_size, hkv, d))
    return dict(q=q, k_pool=k, v_pool=v, qo_indptr=qo_indptr, kv_indptr=kv_indptr,
                kv_page_indices=ids, kv_last_page_len=last, num_qo_heads=hq,
                num_kv_heads=hkv, page_size=page_size)


def visible_range(i, qo_len, kv_len, causal, window_left):
    """Inclusive [lo, hi] from the two inequalities, written as integer bounds."""
    hi = i + kv_len - qo_len if causal else kv_len - 1
    hi = min(hi, kv_len - 1)
    lo = 0 if window_left == -1 else max(0, kv_len + i - qo_len - window_left)
    return lo, hi


# ---------------------------------------------------------------------------
# pin functions (parameterised by the oracle functions so mistakes can be planted)
# ---------------------------------------------------------------------------

def check_golden_masks(mask_fn):
    with open(os.path.join(GOLDEN, "mask_ranges.txt")) as f:
        lines = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(lines) >= 10
    for ln in lines:
        head, rows = ln.split("|")
        qo_len, kv_len, causal, w = (int(t) for t in head.split())
        want = [tuple(int(x) for x in r.split(",")) for r in rows.split()]
        got = mask_fn(qo_len, kv_len, bool(causal), w)
        assert got.shape == (qo_len, kv_len)
        for i, (lo, hi) in enumerate(want):
            expect = np.zeros(kv_len, dtype=bool)
            expect[lo:hi + 1] = True
            assert np.array_equal(got[i], expect), (ln, i, got[i])


def check_golden_attention(attn_fn):
    with open(os.path.join(GOLDEN, "tiny_attention.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        L, P = c["kv_len"], c["page_size"]
        n_pages = (L + P - 1) // P
        k = np.zeros((n_pages, P) + np.shape(c["k"])[1:])
        v = np.zeros((n_pages, P) + np.shape(c["v"])[1:])
        for j in range(L):
            k[j // P, j % P] = c["k"][j]
            v[j // P, j % P] = c["v"][j]
        o, lse = attn_fn(np.array(c["q"], dtype=np.float64), k, v,
                         np.array([0, c["qo_len"]]), np.array([0, n_pages]),
                         np.arange(n_pages), np.array([L - (n_pages - 1) * P]),
                         c["num_qo_heads"], c["num_kv_heads"], P, c["causal"],
                         c["window_left"], c["sm_scale"])
        np.testing.assert_allclose(o, np.array(c["o"]), rtol=0, atol=1e-12, err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-12, err_msg=c["name"])


def check_kv_lengths(kv_len_fn):
    got = kv_len_fn(np.array([0, 2, 2, 5, 6]), np.array([3, 1, 16, 1]), 16)
    assert list(got) == [19, 0, 48, 1]
    assert list(kv_len_fn(np.array([0, 3]), np.array([1]), 1)) == [3]


def check_gather(gather_fn):
    pool = np.zeros((6, 4, 2, 3))
    for p in range(6):
        for s in range(4):
            pool[p, s, :, :] = 100 * p + s
    indptr = np.array([0, 2, 5])
    ids = np.array([4, 1, 0, 5, 2])
    got = gather_fn(pool, indptr, ids, 1, 10, 4)   # request 1: pages 0, 5, 2; 10 keys
    want = [0, 1, 2, 3, 500, 501, 502, 503, 200, 201]
    assert np.array_equal(got[:, 0, 0], want)


def check_closed_form_k_zero(attn_fn, rng):
    """K = 0: every visible score is 0, so lse_i = log(n_i), o_i = mean of visible V."""
    for (qo, kv, causal, w) in [(5, 23, True, -1), (5, 23, True, 3), (7, 19, False, 4),
                                (1, 40, True, 0), (6, 6, True, 2), (9, 4, False, 1)]:
        prob = small_problem(rng, [qo], [kv], 4, 2, 8, 5)
        prob["k_pool"][:] = 0.0
        o, lse = attn_fn(**prob, causal=causal, window_left=w, sm_scale=0.37)
        kb = oracle.gather_request_kv  # only to read V rows back out of the pool
        vb = kb(prob["v_pool"], prob["kv_indptr"], prob["kv_page_indices"], 0, kv, 5)
        for i in range(qo):
            lo, hi = visible_range(i, qo, kv, causal, w)
            n = hi - lo + 1
            for h in range(4):
                assert lse[i, h] == pytest.approx(math.log(n), abs=1e-12)
                want = vb[lo:hi + 1, h // 2, :].mean(axis=0)
                np.testing.assert_allclose(o[i, h], want, atol=1e-12)


def check_v_ones(attn_fn, rng):
    prob = small_problem(rng, [3, 8, 1], [11, 30, 17], 6, 3, 4, 3)
    prob["v_pool"][:] = 1.0
    for causal, w in [(True, -1), (True, 2), (False, 0), (False, -1)]:
        o, _ = attn_fn(**prob, causal=causal, window_left=w, sm_scale=1.3)
        np.testing.assert_allclose(o, 1.0, atol=1e-12)


def check_sdpa(attn_fn, rng):
    """Library routine: torch SDPA (float64, CPU) with a mask made by tril/triu."""
    for (qo, kv, causal, w, hq, hkv) in [(6, 6, True, -1, 2, 2), (5, 17, True, -1, 4, 2),
                                          (5, 17, True, 3, 4, 1), (8, 13, False, 2, 3, 3),
                                          (3, 9, False, -1, 2, 1)]:
        prob = small_problem(rng, [qo], [kv], hq, hkv, 8, 4)
        o, lse = attn_fn(**prob, causal=causal, window_left=w, sm_scale=0.25)
        k = torch.from_numpy(oracle.gather_request_kv(prob["k_pool"], prob["kv_indptr"],
                                                      prob["kv_page_indices"], 0, kv, 4))
        v = torch.from_numpy(oracle.gather_request_kv(prob["v_pool"], prob["kv_indptr"],
                                                      prob["kv_page_indices"], 0, kv, 4))
        q = torch.from_numpy(prob["q"])                          # [qo, hq, d]
        rep = hq // hkv
        k = k.repeat_interleave(rep, dim=1).permute(1, 0, 2)     # [hq, kv, d]
        v = v.repeat_interleave(rep, dim=1).permute(1, 0, 2)
        qh = q.permute(1, 0, 2)
        keep = torch.ones(qo, kv, dtype=torch.bool)
        if causal:   # bottom-right: j - i <= kv - qo
            keep = torch.tril(keep, diagonal=kv - qo)
        if w != -1:  # left band: j - i >= kv - qo - w
            keep = keep & torch.triu(torch.ones(qo, kv, dtype=torch.bool), diagonal=kv - qo - w)
        if causal and w == -1 and qo == kv:
            ref = torch.nn.functional.scaled_dot_product_attention(
                qh, k, v, is_causal=True, scale=0.25)
        else:
            ref = torch.nn.functional.scaled_dot_product_attention(
                qh, k, v, attn_mask=keep, scale=0.25)
        scores = (qh @ k.transpose(1, 2)) * 0.25
        ref_lse = torch.logsumexp(scores.masked_fill(~keep, float("-inf")), dim=-1)
        np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-10)
        np.testing.assert_allclose(lse, ref_lse.permute(1, 0).numpy(), atol=1e-10)


def check_bruteforce_grid(attn_fn, rng, brute_fn=oracle.attention_bruteforce, quick=False):
    heads = [(1, 1), (4, 2), (6, 3)]
    pages = [1, 3, 16]
    n = 0
    for hq, hkv in heads:
        for P in pages:
            B = int(rng.integers(1, 4))
            qo = rng.integers(1, 9, size=B)
            kv = np.maximum(qo, rng.integers(1, 41, size=B))
            prob = small_problem(rng, qo, kv, hq, hkv, 3, P)
            L = int(kv.max())
            for causal in (True, False):
                for w in sorted({-1, 0, 1, max(L - 2, 0), L - 1, L, L + 5}):
                    if quick and n % 5:
                        n += 1
                        continue
                    a = attn_fn(**prob, causal=causal, window_left=w, sm_scale=0.7)
                    bf = brute_fn(**prob, causal=causal, window_left=w, sm_scale=0.7)
                    np.testing.assert_allclose(a[0], bf[0], atol=1e-9)
                    np.testing.assert_allclose(a[1], bf[1], atol=1e-9)
                    n += 1
    return n


# ---------------------------------------------------------------------------
# the tests
# ---------------------------------------------------------------------------

def test_golden_mask_ranges():
    check_golden_masks(oracle.allowed_mask)


def test_golden_tiny_attention():
    check_golden_attention(oracle.attention)
    check_golden_attention(oracle.attention_bruteforce)


def test_kv_lengths_from_paged_metadata():
    check_kv_lengths(oracle.kv_lengths)


def test_gather_follows_page_table():
    check_gather(oracle.gather_request_kv)


def test_bruteforce_matches_vectorised_on_grid():
    assert check_bruteforce_grid(oracle.attention, np.random.default_rng(11)) > 100


def test_closed_form_zero_keys():
    check_closed_form_k_zero(oracle.attention, np.random.default_rng(12))


def test_rows_sum_to_one():
    check_v_ones(oracle.attention, np.random.default_rng(13))


def test_library_sdpa_special_cases():
    check_sdpa(oracle.attention, np.random.default_rng(14))


def test_wide_window_equals_no_window():
    rng = np.random.default_rng(15)
    prob = small_problem(rng, [4, 9], [20, 20], 4, 2, 8, 16)
    base = oracle.attention(**prob, causal=True, window_left=-1, sm_scale=0.3)
    for w in (19, 20, 500):
        got = oracle.attention(**prob, causal=True, window_left=w, sm_scale=0.3)
        np.testing.assert_array_equal(got[0], base[0])
        np.testing.assert_array_equal(got[1], base[1])
    narrower = oracle.attention(**prob, causal=True, window_left=18, sm_scale=0.3)
    assert np.abs(narrower[0] - base[0]).max() > 1e-3


def test_gqa_equals_replicated_kv_heads():
    rng = np.random.default_rng(16)
    prob = small_problem(rng, [5, 3], [12, 30], 6, 2, 8, 4)
    got = oracle.attention(**prob, causal=True, window_left=7, sm_scale=0.4)
    rep = dict(prob)
    rep["k_pool"] = np.repeat(prob["k_pool"], 3, axis=2)
    rep["v_pool"] = np.repeat(prob["v_pool"], 3, axis=2)
    rep["num_kv_heads"] = 6
    want = oracle.attention(**rep, causal=True, window_left=7, sm_scale=0.4)
    np.testing.assert_allclose(got[0], want[0], atol=1e-14)
    np.testing.assert_allclose(got[1], want[1], atol=1e-14)


def test_page_relabelling_is_invisible():
    rng = np.random.default_rng(17)
    prob = small_problem(rng, [5, 7], [33, 18], 4, 4, 8, 4)
    got = oracle.attention(**prob, causal=True, window_left=-1, sm_scale=0.4)
    perm = rng.permutation(prob["k_pool"].shape[0])
    moved = dict(prob)
    moved["k_pool"] = np.empty_like(prob["k_pool"])
    moved["v_pool"] = np.empty_like(prob["v_pool"])
    moved["k_pool"][perm] = prob["k_pool"]
    moved["v_pool"][perm] = prob["v_pool"]
    moved["kv_page_indices"] = perm[prob["kv_page_indices"]]
    want = oracle.attention(**moved, causal=True, window_left=-1, sm_scale=0.4)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])


def test_last_verify_row_equals_decode():
    rng = np.random.default_rng(18)
    prob = small_problem(rng, [4, 4, 4], [9, 40, 17], 8, 2, 8, 16)
    o, lse = oracle.attention(**prob, causal=True, window_left=-1, sm_scale=0.5)
    dec = dict(prob)
    dec["q"] = prob["q"][[3, 7, 11]]
    dec["qo_indptr"] = np.arange(4)
    od, lsed = oracle.attention(**dec, causal=True, window_left=-1, sm_scale=0.5)
    np.testing.assert_allclose(o[[3, 7, 11]], od, atol=1e-14)
    np.testing.assert_allclose(lse[[3, 7, 11]], lsed, atol=1e-14)


@pytest.mark.parametrize("causal,w", [(True, -1), (True, 13), (False, 5), (False, -1)])
def test_split_then_merge_equals_unsplit(causal, w):
    rng = np.random.default_rng(19)
    prob = small_problem(rng, [6, 1, 9], [50, 37, 64], 4, 2, 8, 16)
    whole = oracle.attention(**prob, causal=causal, window_left=w, sm_scale=0.4)
    bounds = [0, 7, 16, 16, 40, 64]
    parts = [oracle.attention(**prob, causal=causal, window_left=w, sm_scale=0.4,
                              kv_begin=a, kv_end=e) for a, e in zip(bounds[:-1], bounds[1:])]
    o, lse = oracle.merge_many([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, whole[0], atol=1e-12)
    np.testing.assert_allclose(lse, whole[1], atol=1e-12)
    # an empty chunk is (0, -inf)
    empty = parts[2]
    assert np.all(np.isneginf(empty[1])) and np.all(empty[0] == 0)


def test_merge_algebra():
    rng = np.random.default_rng(20)
    o = [rng.standard_normal((5, 3, 4)) for _ in range(3)]
    lse = [rng.standard_normal((5, 3)) * 4 for _ in range(3)]
    ab = oracle.merge_states(o[0], lse[0], o[1], lse[1])
    ba = oracle.merge_states(o[1], lse[1], o[0], lse[0])
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-14)
    np.testing.assert_allclose(ab[1], ba[1], atol=1e-14)
    left = oracle.merge_states(*ab, o[2], lse[2])
    bc = oracle.merge_states(o[1], lse[1], o[2], lse[2])
    right = oracle.merge_states(o[0], lse[0], *bc)
    np.testing.assert_allclose(left[0], right[0], atol=1e-12)
    np.testing.assert_allclose(left[1], right[1], atol=1e-12)
    # closed form: two equal states merge to themselves with lse + log 2
    same = oracle.merge_states(o[0], lse[0], o[0], lse[0])
    np.testing.assert_allclose(same[0], o[0], atol=1e-14)
    np.testing.assert_allclose(same[1], lse[0] + math.log(2), atol=1e-14)
    # -inf is the identity, exactly; two -inf give (0, -inf)
    ninf = np.full((5, 3), -np.inf)
    idn = oracle.merge_states(o[0], lse[0], np.zeros_like(o[0]), ninf)
    np.testing.assert_array_equal(idn[0], o[0])
    np.testing.assert_array_equal(idn[1], lse[0])
    both = oracle.merge_states(o[0], ninf, o[1], ninf)
    assert np.all(both[0] == 0) and np.all(np.isneginf(both[1]))


def test_non_vacuity_on_workloads():
    """Windowed vs unwindowed, causal vs not, and a wrong GQA map all differ by > 0.1."""
    w = workloads.config1(window_left=31)
    q, k, v = w.float_inputs()
    args = w.plan_args()
    del args["head_dim"]
    base = oracle.attention(q, k, v, **{**args, "window_left": -1})
    win = oracle.attention(q, k, v, **args)
    nonc = oracle.attention(q, k, v, **{**args, "window_left": -1, "causal": False})
    assert np.abs(base[0] - win[0]).max() > 0.1
    assert np.abs(base[0] - nonc[0]).max() > 0.1
    # wrong GQA mapping: interleaved (h % Hkv) instead of consecutive groups
    k_swapped = k[:, :, ::-1, :].copy()
    v_swapped = v[:, :, ::-1, :].copy()
    wrong = oracle.attention(q, k_swapped, v_swapped, **{**args, "window_left": -1})
    assert np.abs(base[0] - wrong[0]).max() > 0.1


def test_refuses_indivisible_heads():
    rng = np.random.default_rng(21)
    prob = small_problem(rng, [2], [4], 4, 4, 4, 2)
    prob["num_qo_heads"], prob["num_kv_heads"] = 12, 8
    with pytest.raises(ValueError):
        oracle.attention(**prob, causal=True, window_left=-1, sm_scale=1.0)


# ---------------------------------------------------------------------------
# planted mistakes: every pin family must reject a plausible wrong oracle
# ---------------------------------------------------------------------------

def _top_left_causal(qo_len, kv_len, causal, window_left, kv_begin=None, kv_end=None):
    m = oracle.allowed_mask(qo_len, kv_len, False, window_left, kv_begin, kv_end)
    if causal:
        i = np.arange(qo_len)[:, None]
        j = np.arange(kv_len)[None, :]
        m &= j <= i
    return m


def _window_off_by_one(qo_len, kv_len, causal, window_left, kv_begin=None, kv_end=None):
    w = window_left if window_left == -1 else window_left + 1
    return oracle.allowed_mask(qo_len, kv_len, causal, w, kv_begin, kv_end)


def _with_mask(mask_fn):
    def attn(*a, **kw):
        saved = oracle.attention.__globals__["allowed_mask"]
        oracle.attention.__globals__["allowed_mask"] = mask_fn
        try:
            return oracle.attention(*a, **kw)
        finally:
            oracle.attention.__globals__["allowed_mask"] = saved
    return attn


def _scale_dropped(*a, **kw):
    a = list(a)
    if "sm_scale" in kw:
        kw["sm_scale"] = 1.0
    elif len(a) > 12:
        a[12] = 1.0
    return oracle.attention(*a, **kw)


def _log2_lse(*a, **kw):
    o, lse = oracle.attention(*a, **kw)
    return o, lse / math.log(2)


def _interleaved_gqa(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_page_indices,
                     kv_last_page_len, num_qo_heads, num_kv_heads, page_size, causal,
                     window_left, sm_scale, **kw):
    # q head h reads kv head h % Hkv instead of h // group
    group = num_qo_heads // num_kv_heads
    order = [(h % num_kv_heads) * group + h // num_kv_heads for h in range(num_qo_heads)]
    inv = np.argsort(order)
    o, lse = oracle.attention(np.asarray(q)[:, order], k_pool, v_pool, qo_indptr,
                              kv_indptr, kv_page_indices, kv_last_page_len,
                              num_qo_heads, num_kv_heads, page_size, causal,
                              window_left, sm_scale, **kw)
    return o[:, inv], lse[:, inv]


def _slot_from_wrong_page(pool, kv_indptr, kv_page_indices, b, kv_len, page_size):
    # uses the logical page number instead of the page table
    rows = [pool[j // page_size, j % page_size] for j in range(int(kv_len))]
    return np.stack(rows).astype(np.float64) if rows else np.zeros((0,) + pool.shape[2:])


def _transposed_pv(*a, **kw):
    o, lse = oracle.attention(*a, **kw)
    return o[..., ::-1], lse


@pytest.mark.parametrize("name", ["top_left_causal", "window_off_by_one", "scale_dropped",
                                  "log2_lse", "interleaved_gqa", "wrong_page",
                                  "reversed_head_dim"])
def test_pins_reject_planted_mistakes(name):
    rng = np.random.default_rng(22)

    def fails(check, *args):
        try:
            check(*args)
        except AssertionError:
            return True
        return False

    if name == "top_left_causal":
        assert fails(check_golden_masks, _top_left_causal)
        assert fails(check_sdpa, _with_mask(_top_left_causal), rng)
    elif name == "window_off_by_one":
        assert fails(check_golden_masks, _window_off_by_one)
        assert fails(check_closed_form_k_zero, _with_mask(_window_off_by_one), rng)
    elif name == "scale_dropped":
        assert fails(check_golden_attention, _scale_dropped)
        assert fails(check_sdpa, _scale_dropped, rng)
    elif name == "log2_lse":
        assert fails(check_golden_attention, _log2_lse)
        assert fails(check_closed_form_k_zero, _log2_lse, rng)
    elif name == "interleaved_gqa":
        assert fails(check_golden_attention, _interleaved_gqa) or \
            fails(check_sdpa, _interleaved_gqa, rng)
        assert fails(check_sdpa, _interleaved_gqa, rng)
    elif name == "wrong_page":
        assert fails(check_gather, _slot_from_wrong_page)
    elif name == "reversed_head_dim":
        assert fails(check_golden_attention, _transposed_pv)
        assert fails(check_sdpa, _transposed_pv, rng)


def test_sampled_rows_match_full_oracle():
    rng = np.random.default_rng(23)
    prob = small_problem(rng, [6, 9], [30, 12], 6, 2, 8, 4)
    for causal, w in [(True, -1), (True, 3), (False, 2)]:
        full = oracle.attention(**prob, causal=causal, window_left=w, sm_scale=0.6)
        for b, rows in ((0, [0, 5, 2]), (1, [8, 0])):
            heads = [5, 0, 3]
            o, lse = oracle.attention_rows(**prob, causal=causal, window_left=w, sm_scale=0.6,
                                           b=b, rows=rows, heads=heads)
            base = int(prob["qo_indptr"][b])
            for ri, i in enumerate(rows):
                for hi, h in enumerate(heads):
                    np.testing.assert_allclose(o[ri, hi], full[0][base + i, h], atol=1e-12)
                    assert lse[ri, hi] == pytest.approx(full[1][base + i, h], abs=1e-12)
    # restricted key range matches the full oracle's partial state
    part = oracle.attention(**prob, causal=True, window_left=-1, sm_scale=0.6, kv_begin=4, kv_end=9)
    o, lse = oracle.attention_rows(**prob, causal=True, window_left=-1, sm_scale=0.6, b=1,
                                   rows=[0, 8], heads=[1], kv_begin=4, kv_end=9)
    np.testing.assert_allclose(o[:, 0], part[0][[6, 14], 1], atol=1e-12)


def test_append_hand_example():
    """Two requests, page size 2: hand-placed destinations of three new tokens."""
    pool = np.zeros((4, 2, 1, 1))
    indptr = np.array([0, 2, 3])
    pages = np.array([3, 0, 2])        # request 0: pages 3, 0; request 1: page 2
    ak = np.array([[[1.0]], [[2.0]], [[3.0]]])
    av = -ak
    # token 0 -> request 0 pos 2 -> page 0 slot 0; token 1 -> request 0 pos 1 -> page 3 slot 1;
    # token 2 -> request 1 pos 1 -> page 2 slot 1
    k, v = oracle.append_paged_kv(pool, pool, ak, av, [0, 0, 1], [2, 1, 1], indptr, pages, 2)
    want = np.zeros((4, 2))
    want[0, 0], want[3, 1], want[2, 1] = 1.0, 2.0, 3.0
    np.testing.assert_array_equal(k[:, :, 0, 0], want)
    np.testing.assert_array_equal(v[:, :, 0, 0], -want)
    assert np.all(pool == 0)           # input untouched


def test_append_then_gather_round_trip():
    rng = np.random.default_rng(30)
    prob = small_problem(rng, [3, 5], [20, 33], 4, 2, 8, 16)
    L = oracle.kv_lengths(prob["kv_indptr"], prob["kv_last_page_len"], 16)
    # append the last 4 and 7 keys of the two requests
    bi = np.array([0] * 4 + [1] * 7)
    pos = np.concatenate([np.arange(L[0] - 4, L[0]), np.arange(L[1] - 7, L[1])])
    ak = rng.standard_normal((11, 2, 8))
    av = rng.standard_normal((11, 2, 8))
    k, v = oracle.append_paged_kv(prob["k_pool"], prob["v_pool"], ak, av, bi, pos,
                                  prob["kv_indptr"], prob["kv_page_indices"], 16)
    for b, (lo, n) in enumerate([(0, 4), (4, 7)]):
        kb = oracle.gather_request_kv(k, prob["kv_indptr"], prob["kv_page_indices"], b, L[b], 16)
        old = oracle.gather_request_kv(prob["k_pool"], prob["kv_indptr"], prob["kv_page_indices"],
                                       b, L[b], 16)
        np.testing.assert_array_equal(kb[L[b] - n:], ak[lo:lo + n])
        np.testing.assert_array_equal(kb[:L[b] - n], old[:L[b] - n])
    # slots no token targets are unchanged
    touched = np.zeros(prob["k_pool"].shape[:2], dtype=bool)
    for t in range(11):
        b = bi[t]
        page = prob["kv_page_indices"][prob["kv_indptr"][b] + pos[t] // 16]
        touched[page, pos[t] % 16] = True
    np.testing.assert_array_equal(k[~touched], prob["k_pool"][~touched])


# ---------------------------------------------------------------------------
# custom (tree-draft topology) masks
# ---------------------------------------------------------------------------
def _tree_golden():
    with open(os.path.join(GOLDEN, "tree_mask.json")) as f:
        return json.load(f)


def test_custom_mask_golden_bits():
    g = _tree_golden()
    want = np.array(g["mask"], dtype=bool)
    got = oracle.custom_mask_rows(np.array(g["packed_bytes"], np.uint8), [0, 3], 0,
                                  g["qo_len"], g["kv_len"])
    assert np.array_equal(got, want)
    # the input encoder used by the tests agrees with the hand-packed bytes
    data, indptr = W.pack_custom_mask([W.tree_topology_mask(g["prefix_len"], g["parents"])])
    assert list(data) == g["packed_bytes"] and list(indptr) == [0, 3]


def test_custom_mask_golden_attention():
    """K = 0 makes every visible score equal: lse = log(#visible) and o = the
    mean of the visible V rows (V row j = j)."""
    g = _tree_golden()
    Q, L = g["qo_len"], g["kv_len"]
    q = np.ones((Q, 1, 1))
    k = np.zeros((2, 4, 1, 1))                       # two pages of 4 keys
    v = np.arange(8, dtype=np.float64).reshape(2, 4, 1, 1)
    o, lse = oracle.attention(q, k, v, [0, Q], [0, 2], [0, 1], [2], 1, 1, 4, False, -1, 1.0,
                              custom_mask=np.array(g["packed_bytes"], np.uint8),
                              mask_indptr=[0, 3])
    assert np.allclose(lse[:, 0], np.log(g["visible_counts"]), atol=1e-12)
    assert np.allclose(o[:, 0, 0], g["mean_of_key_index"], atol=1e-12)


def _tree_case(rng, qo_trees, prefixes, hq, hkv, d, page, window):
    mats = [W.tree_topology_mask(p, W.random_tree_parents(rng, n))
            for n, p in zip(qo_trees, prefixes)]
    kv = [p + n for n, p in zip(qo_trees, prefixes)]
    w = W.build("tree", qo_trees, kv, hq, hkv, d, page, False, window, W.FP16,
                seed=int(rng.integers(1 << 30)))
    w.custom_mask, w.mask_indptr = W.pack_custom_mask(mats)
    return w, mats


def test_custom_mask_matches_bruteforce():
    rng = np.random.default_rng(61)
    for trial in range(6):
        w, _ = _tree_case(rng, [int(x) for x in rng.integers(1, 7, size=2)],
                          [int(x) for x in rng.integers(0, 9, size=2)], 4, 2, 8,
                          int(rng.choice([1, 3, 4])), int(rng.choice([-1, 0, 2, 5])))
        q, k, v = w.float_inputs()
        a = w.plan_args()
        del a["head_dim"]
        o1, l1 = oracle.attention(q, k, v, **a)
        o2, l2 = oracle.attention_bruteforce(q, k, v, **a)
        assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)


def test_custom_mask_reduces_to_causal_and_full():
    rng = np.random.default_rng(62)
    w = W.build("m", [5, 3], [9, 3], 4, 2, 8, 4, True, -1, W.FP16, seed=63)
    q, k, v = w.float_inputs()
    a = w.plan_args()
    del a["head_dim"]
    ref_c = oracle.attention(q, k, v, **a)
    a_nc = {**a, "causal": False}
    ref_n = oracle.attention(q, k, v, **a_nc)
    causal_mats = [oracle.allowed_mask(int(ql), int(kl), True, -1)
                   for ql, kl in zip(w.qo_lens, w.kv_lens)]
    data, ind = W.pack_custom_mask(causal_mats)
    got_c = oracle.attention(q, k, v, **a_nc, custom_mask=data, mask_indptr=ind)
    data, ind = W.pack_custom_mask([np.ones((int(ql), int(kl)), bool)
                                    for ql, kl in zip(w.qo_lens, w.kv_lens)])
    got_n = oracle.attention(q, k, v, **a_nc, custom_mask=data, mask_indptr=ind)
    for (o1, l1), (o2, l2) in ((ref_c, got_c), (ref_n, got_n)):
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # a chain (each node's parent is the previous one) is exactly causal verify
    mats = [W.tree_topology_mask(int(kl) - int(ql), np.arange(int(ql)) - 1)
            for ql, kl in zip(w.qo_lens, w.kv_lens)]
    data, ind = W.pack_custom_mask(mats)
    got = oracle.attention(q, k, v, **a_nc, custom_mask=data, mask_indptr=ind)
    assert np.array_equal(got[0], ref_c[0]) and np.array_equal(got[1], ref_c[1])
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, **a, custom_mask=data, mask_indptr=ind)


def test_custom_mask_tree_differs_from_causal():
    """Non-vacuity: a branching tree must not give the causal answer (a causal
    mask lets a draft token see its sibling branch)."""
    rng = np.random.default_rng(64)
    w, mats = _tree_case(rng, [6], [5], 2, 1, 8, 4, -1)
    parents_branch = W.tree_topology_mask(5, [-1, 0, 0, 1, 1, 2])
    w.custom_mask, w.mask_indptr = W.pack_custom_mask([parents_branch])
    q, k, v = w.float_inputs()
    a = w.plan_args()
    del a["head_dim"]
    o_t, _ = oracle.attention(q, k, v, **a)
    a_c = {x: y for x, y in a.items() if x not in ("custom_mask", "mask_indptr")}
    o_c, _ = oracle.attention(q, k, v, **{**a_c, "causal": True})
    assert np.abs(o_t - o_c).max() > 0.1


def test_custom_mask_rows_match_full():
    rng = np.random.default_rng(65)
    w, _ = _tree_case(rng, [7, 4, 9], [40, 3, 70], 8, 2, 16, 16, 30)
    q, k, v = w.float_inputs()
    a = w.plan_args()
    del a["head_dim"]
    o, lse = oracle.attention(q, k, v, **a)
    for b in range(3):
        rows = list(range(int(w.qo_lens[b])))
        heads = [0, 5, 7]
        o_r, l_r = oracle.attention_rows(q, k, v, **a, b=b, rows=rows, heads=heads)
        q0 = int(w.qo_indptr[b])
        assert np.allclose(o_r, o[q0:q0 + len(rows)][:, heads], atol=1e-12)
        assert np.allclose(l_r, lse[q0:q0 + len(rows)][:, heads], atol=1e-12)


# ---------------------------------------------------------------------------
# logits soft-cap
# ---------------------------------------------------------------------------
def test_soft_cap_golden():
    with open(os.path.join(GOLDEN, "soft_cap.json")) as f:
        g = json.load(f)
    q = np.ones((1, 1, 1))
    k = np.array(g["raw_dot"], dtype=np.float64).reshape(1, 2, 1, 1)
    v = np.array(g["v"], dtype=np.float64).reshape(1, 2, 1, 1)
    o, lse = oracle.attention(q, k, v, [0, 1], [0, 1], [0], [2], 1, 1, 2, False, -1,
                              g["sm_scale"], logits_soft_cap=g["cap"])
    assert abs(lse[0, 0] - g["lse"]) < 1e-12 and abs(o[0, 0, 0] - g["o"]) < 1e-12
    ob, lb = oracle.attention_bruteforce(q, k, v, [0, 1], [0, 1], [0], [2], 1, 1, 2, False, -1,
                                         g["sm_scale"], logits_soft_cap=g["cap"])
    assert abs(lb[0, 0] - g["lse"]) < 1e-12 and abs(ob[0, 0, 0] - g["o"]) < 1e-12


def test_soft_cap_bounds_limit_and_bruteforce():
    w = W.build("cap", [6, 3], [20, 9], 4, 2, 8, 4, True, 5, W.FP16, seed=91)
    q, k, v = w.float_inputs()
    a = w.plan_args()
    del a["head_dim"]
    base = oracle.attention(q, k, v, **a)
    # a cap far above every logit changes nothing measurable
    far = oracle.attention(q, k, v, **a, logits_soft_cap=1e9)
    assert np.allclose(far[0], base[0], atol=1e-12) and np.allclose(far[1], base[1], atol=1e-12)
    # brute force agrees at a biting cap
    big = {**a, "sm_scale": 40.0}
    o1, l1 = oracle.attention(q, k, v, **big, logits_soft_cap=2.0)
    o2, l2 = oracle.attention_bruteforce(q, k, v, **big, logits_soft_cap=2.0)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)
    # every capped logit lies in (-cap, cap): lse within log(#visible) +- cap
    counts = np.concatenate([oracle.allowed_mask(int(ql), int(kl), True, 5).sum(1)
                             for ql, kl in zip(w.qo_lens, w.kv_lens)])
    assert (l1 <= 2.0 + np.log(counts)[:, None] + 1e-12).all()
    assert (l1 >= -2.0 + np.log(counts)[:, None] - 1e-12).all()
    # and the cap bites: the uncapped scores at that scale differ
    o3, _ = oracle.attention(q, k, v, **big)
    assert np.abs(o3 - o1).max() > 0.1


# ---------------------------------------------------------------------------
# FP8 E4M3 K/V
# ---------------------------------------------------------------------------
def test_e4m3_golden_codes():
    with open(os.path.join(GOLDEN, "e4m3.json")) as f:
        g = json.load(f)
    got = oracle.decode_e4m3(np.array(g["codes"], np.uint8))
    assert np.array_equal(got, np.array(g["values"])), got
    assert np.signbit(got[1])
    assert np.isnan(oracle.decode_e4m3(np.array(g["nan_codes"], np.uint8))).all()
    assert np.array_equal(oracle.decode_e4m3(np.array(g["codes"], np.uint8), 0.5),
                          np.array(g["values"]) * 0.5)


def test_e4m3_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_attention_over_e4m3_pools_is_attention_over_their_values():
    w = W.build("fp8", [5, 9], [33, 40], 4, 2, 16, 8, True, -1, W.BF16, seed=95)
    rng = np.random.default_rng(96)
    kc = torch.from_numpy(rng.standard_normal(w.k_pool.shape).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    vc = torch.from_numpy(rng.standard_normal(w.v_pool.shape).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    q, _, _ = w.float_inputs()
    a = w.plan_args()
    del a["head_dim"]
    kf, vf = oracle.decode_e4m3(kc, 0.25), oracle.decode_e4m3(vc, 3.0)
    o, lse = oracle.attention(q, kf, vf, **a)
    o2, lse2 = oracle.attention_bruteforce(q, kf, vf, **a)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)
    # the V scale scales o only; the K scale enters the logits
    o3, lse3 = oracle.attention(q, kf, oracle.decode_e4m3(vc, 1.0), **a)
    assert np.allclose(o, 3.0 * o3, atol=1e-12) and np.array_equal(lse, lse3)
