"""Plain CPU oracle for batched attention prefill over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, helpers, tables or constants) and imports nothing from it.

Everything here is the plain definition written out, in float64, with NumPy
matmul / exp / log as the only library steps:

* ``kv_lengths``        -- per-request key count from the paged metadata.
* ``gather_request_kv`` -- logical K/V rows of one request through its page table.
* ``allowed_mask``      -- bottom-right causal mask and left-only window.
* ``attention``         -- masked softmax(sm_scale * Q K^T) V with GQA, plus LSE.
* ``attention_bruteforce`` -- the same definition as per-element Python loops.
* ``merge_states`` / ``merge_many`` -- combining partial (o, lse) states.
* ``append_paged_kv``   -- writing new K/V rows into their pages.
* ``custom_mask_rows``  -- a request's topology mask (tree drafts) from packed bits.
* ``soft_cap``          -- the logits soft-cap transform.
* ``decode_e4m3``       -- FP8 E4M3 cache bytes to values (times a per-tensor scale).

Sources (web pages of the AMD-Ecosystem FlashInfer fork):
  [W]  PR #339 "Route non-causal windowed prefill to AITER's masked kernel",
       section "Why window_size_right stays -1" (left-only, bottom-right
       anchored band, applied independently of causal).
  [C]  PR #362 "Support speculative-decode verify on ROCm, and stop auto
       routing short-query prefill to AITER", Summary and the verify commit
       message (the ROCm causal mask is bottom-right aligned: the last query
       row attends to the whole KV).
  [K]  PR #362, Review notes (kv_len is derived from indptr and
       last_page_len, not from a caller's seq_lens).
  [G]  PR #399 "Refuse attention inputs the ROCm kernels would compute
       wrongly", What changed / GQA head divisibility.
  [M]  PR #399, What changed / Graph-mode partial_state merge, and PR #362's
       split-KV test commit (partial (o, lse) states merged into one result).
  [T]  PR #362, Architecture / design notes: a causal mask verifies chain
       drafts only; tree drafts need a topology mask (custom_mask).
  [S]  PR #362, Architecture / design notes and per-commit messages: a
       logits soft-cap exists and a route that ignores it gives a wrong
       answer (the pages gate on it but do not give the formula).
  [F]  PR #362, per-commit messages (the merge with the fp8 branch): fp8
       prefill exists on the in-tree paged route (the pages do not give the
       format).

Readings where the pages are silent (each also listed in the design notes):
  * kv_len = (n_pages - 1) * page_size + last_page_len, 0 for no pages.
  * logical key j of a request sits at page indices[indptr[b] + j // P],
    slot j % P, in an NHD pool [num_pages, P, Hkv, D].
  * causal keeps j <= i + kv_len - qo_len (bottom-right).
  * GQA: q head h reads kv head h // (Hq // Hkv) (consecutive groups).
  * lse uses the natural logarithm.
  * a row with no visible key has o = 0 and lse = -inf (only reachable for a
    partial state restricted to a key range, or a custom mask).
  * custom mask [T]: request b's mask is the row-major [qo_len, kv_len]
    boolean matrix (query i, key j) -> bit i * kv_len + j, packed
    little-endian (bit k sits in byte k // 8 at bit k % 8) from byte
    mask_indptr[b].  It replaces the causal mask (causal must be off); the
    left window still applies on top of it.
  * logits soft-cap [S]: with cap > 0 every scaled logit s becomes
    cap * tanh(s / cap) before the softmax (cap = 0: no cap).
  * fp8 K/V [F]: the OCP FP8 E4M3 format (sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 subnormal; S.1111.111 NaN; no infinities),
    each cache multiplied by a per-tensor float scale.
Parity status: every function here is pinned by tests/test_oracle_pins.py
(brute force, closed forms, library routines, invariants, golden fixtures).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


def kv_lengths(kv_indptr, kv_last_page_len, page_size):
    """Per-request key count from the paged metadata [K].

    A request with n >= 1 pages holds (n - 1) full pages plus last_page_len
    keys on its final page; a request with no page holds no key.
    """
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(kv_last_page_len, dtype=np.int64)
    n_pages = kv_indptr[1:] - kv_indptr[:-1]
    return np.where(n_pages > 0, (n_pages - 1) * page_size + last, 0)


def gather_request_kv(pool, kv_indptr, kv_page_indices, b, kv_len, page_size):
    """Logical rows [kv_len, Hkv, D] of request b from an NHD page pool.

    Logical key j lives on physical page kv_page_indices[kv_indptr[b] + j // P]
    at slot j % P (the paged-KV page table the pages describe for paged_kv_t).
    """
    first = int(kv_indptr[b])
    rows = []
    for j in range(int(kv_len)):
        page = int(kv_page_indices[first + j // page_size])
        rows.append(pool[page, j % page_size])
    if not rows:
        return np.zeros((0,) + pool.shape[2:], dtype=np.float64)
    return np.stack(rows).astype(np.float64)


def allowed_mask(qo_len, kv_len, causal, window_left, kv_begin=None, kv_end=None):
    """Boolean [qo_len, kv_len]: may query row i attend to key j?

    causal [C]: bottom-right aligned, j <= i + kv_len - qo_len.
    window [W]: left-only band, applied independently of causal,
                j + qo_len + window_left >= kv_len + i;  window_left = -1
                means no window.
    kv_begin/kv_end restrict the keys to [kv_begin, kv_end) in the request's
    own (global) key coordinates, which is what one split-KV chunk sees [M].
    """
    i = np.arange(qo_len, dtype=np.int64)[:, None]
    j = np.arange(kv_len, dtype=np.int64)[None, :]
    ok = np.ones((qo_len, kv_len), dtype=bool)
    if causal:
        ok &= j <= i + kv_len - qo_len
    if window_left != -1:
        ok &= j + qo_len + window_left >= kv_len + i
    if kv_begin is not None:
        ok &= j >= kv_begin
    if kv_end is not None:
        ok &= j < kv_end
    return ok


def soft_cap(s, cap):
    """cap * tanh(s / cap) for cap > 0, s unchanged for cap = 0 [S]."""
    if cap is None or cap == 0:
        return s
    if not cap > 0:
        raise ValueError(f"logits_soft_cap: expected >= 0, given {cap}")
    return cap * np.tanh(np.asarray(s, dtype=np.float64) / cap)


def decode_e4m3(codes, scale=1.0):
    """Values of FP8 E4M3 codes (uint8 array), times scale [F].

    value = (-1)^s * 2^(e - 7) * (1 + m / 8) for exponent field e in 1..15
    (except e = 15, m = 7: NaN), and (-1)^s * 2^-6 * (m / 8) for e = 0.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, -6)
    v = sign * np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return v * float(scale)


def custom_mask_rows(custom_mask, mask_indptr, b, qo_len, kv_len):
    """Boolean [qo_len, kv_len] topology mask of request b from packed bits [T].

    Bit i * kv_len + j (little-endian within each byte, request b's bits from
    byte mask_indptr[b]) says whether query row i may attend key j.
    """
    start = int(mask_indptr[b])
    n = int(qo_len) * int(kv_len)
    nbytes = (n + 7) // 8
    seg = np.asarray(custom_mask[start:start + nbytes], dtype=np.uint8)
    if seg.size != nbytes:
        raise ValueError(f"custom_mask: request {b} needs {nbytes} bytes from {start}")
    bits = np.unpackbits(seg, bitorder="little")[:n]
    return bits.reshape(int(qo_len), int(kv_len)).astype(bool)


def _check_custom(custom_mask, mask_indptr, causal):
    if custom_mask is None:
        return False
    if mask_indptr is None:
        raise ValueError("custom_mask needs mask_indptr")
    if causal:
        raise ValueError("a custom mask replaces the causal mask: pass causal=False")
    return True


def _check_heads(num_qo_heads, num_kv_heads):
    # [G]: a group size that does not divide the head count is refused.
    if num_kv_heads <= 0 or num_qo_heads % num_kv_heads != 0:
        raise ValueError("num_qo_heads must be a positive multiple of num_kv_heads")


def attention(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_page_indices,
              kv_last_page_len, num_qo_heads, num_kv_heads, page_size, causal,
              window_left, sm_scale, kv_begin=None, kv_end=None, custom_mask=None,
              mask_indptr=None, logits_soft_cap=0.0):
    """Masked softmax attention over a paged KV cache, in float64.

    q: [total_q, Hq, D]; k_pool, v_pool: NHD [num_pages, P, Hkv, D].
    Returns o [total_q, Hq, D] and lse [total_q, Hq] (natural log), both float64.
    For every request b, q head h, row i:
        s_ij  = sm_scale * <q_i,h , K_b[j, h // group]>      over allowed j
        lse_i = log sum_j exp(s_ij)
        o_i   = sum_j exp(s_ij - lse_i) * V_b[j, h // group]
    A row with no allowed key gets o = 0, lse = -inf.
    kv_begin/kv_end (optional) restrict every request to keys in that range of
    its own key coordinates, giving the partial state of one KV chunk.
    custom_mask/mask_indptr (optional, packed bits [T]) intersect the mask with
    each request's topology mask; logits_soft_cap > 0 caps every s_ij [S].
    """
    _check_heads(num_qo_heads, num_kv_heads)
    use_custom = _check_custom(custom_mask, mask_indptr, causal)
    group = num_qo_heads // num_kv_heads
    q = np.asarray(q, dtype=np.float64)
    total_q, hq, d = q.shape
    assert hq == num_qo_heads
    o = np.zeros((total_q, hq, d), dtype=np.float64)
    lse = np.full((total_q, hq), NEG_INF, dtype=np.float64)
    kv_len = kv_lengths(kv_indptr, kv_last_page_len, page_size)
    for b in range(len(kv_len)):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        qo_len, L = q1 - q0, int(kv_len[b])
        if qo_len == 0:
            continue
        kb = gather_request_kv(k_pool, kv_indptr, kv_page_indices, b, L, page_size)
        vb = gather_request_kv(v_pool, kv_indptr, kv_page_indices, b, L, page_size)
        mask = allowed_mask(qo_len, L, causal, window_left, kv_begin, kv_end)
        if use_custom:
            mask = mask & custom_mask_rows(custom_mask, mask_indptr, b, qo_len, L)
        has_key = mask.any(axis=1)
        for h in range(hq):
            g = h // group
            s = soft_cap(sm_scale * (q[q0:q1, h, :] @ kb[:, g, :].T), logits_soft_cap)
            s = np.where(mask, s, NEG_INF)
            m = np.max(s, axis=1, initial=NEG_INF)
            m_safe = np.where(has_key, m, 0.0)
            e = np.where(mask, np.exp(s - m_safe[:, None]), 0.0)
            total = e.sum(axis=1)
            row_lse = np.where(has_key, m_safe + np.log(np.where(has_key, total, 1.0)), NEG_INF)
            p = e / np.where(has_key, total, 1.0)[:, None]
            o[q0:q1, h, :] = p @ vb[:, g, :]
            lse[q0:q1, h] = row_lse
    return o, lse


def attention_bruteforce(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_page_indices,
                         kv_last_page_len, num_qo_heads, num_kv_heads, page_size,
                         causal, window_left, sm_scale, kv_begin=None, kv_end=None,
                         custom_mask=None, mask_indptr=None, logits_soft_cap=0.0):
    """The same definition as ``attention`` as literal per-element loops.

    Pure Python floats (IEEE double), no NumPy arithmetic: for tiny inputs only.
    Every key's page and slot, the mask predicate and the GQA head are
    evaluated per (request, head, row, key).
    """
    _check_heads(num_qo_heads, num_kv_heads)
    use_custom = _check_custom(custom_mask, mask_indptr, causal)
    group = num_qo_heads // num_kv_heads
    total_q, hq, d = np.shape(q)
    o = [[[0.0] * d for _ in range(hq)] for _ in range(total_q)]
    lse = [[NEG_INF] * hq for _ in range(total_q)]
    batch = len(kv_indptr) - 1
    for b in range(batch):
        n_pages = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        L = 0 if n_pages == 0 else (n_pages - 1) * page_size + int(kv_last_page_len[b])
        qo_len = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        for h in range(hq):
            g = h // group
            for i in range(qo_len):
                row = int(qo_indptr[b]) + i
                scores, values = [], []
                for j in range(L):
                    ok = True
                    if causal and not (j <= i + L - qo_len):
                        ok = False
                    if window_left != -1 and not (j + qo_len + window_left >= L + i):
                        ok = False
                    if kv_begin is not None and j < kv_begin:
                        ok = False
                    if kv_end is not None and j >= kv_end:
                        ok = False
                    if use_custom:
                        bit = i * L + j
                        byte = int(custom_mask[int(mask_indptr[b]) + bit // 8])
                        if (byte >> (bit % 8)) & 1 == 0:
                            ok = False
                    if not ok:
                        continue
                    page = int(kv_page_indices[int(kv_indptr[b]) + j // page_size])
                    slot = j % page_size
                    dot = 0.0
                    for t in range(d):
                        dot += float(q[row][h][t]) * float(k_pool[page][slot][g][t])
                    sc = sm_scale * dot
                    if logits_soft_cap:
                        sc = logits_soft_cap * math.tanh(sc / logits_soft_cap)
                    scores.append(sc)
                    values.append([float(v_pool[page][slot][g][t]) for t in range(d)])
                if not scores:
                    continue
                m = max(scores)
                denom = sum(math.exp(s - m) for s in scores)
                row_lse = m + math.log(denom)
                acc = [0.0] * d
                for s, v in zip(scores, values):
                    w = math.exp(s - row_lse)
                    for t in range(d):
                        acc[t] += w * v[t]
                o[row][h] = acc
                lse[row][h] = row_lse
    return np.array(o, dtype=np.float64).reshape(total_q, hq, d), \
        np.array(lse, dtype=np.float64).reshape(total_q, hq)


def merge_states(o_a, lse_a, o_b, lse_b):
    """Combine two partial states over disjoint key sets [M].

    If (o_x, lse_x) is softmax attention over key set X, the state over
    A u B is: lse = log(exp(lse_a) + exp(lse_b)),
              o   = (exp(lse_a) o_a + exp(lse_b) o_b) / exp(lse).
    Computed relative to the larger lse; two empty states give (0, -inf).
    o: [..., D], lse: [...], float64.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w_a = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - m_safe))
    w_b = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - m_safe))
    total = w_a + w_b
    denom = np.where(empty, 1.0, total)
    o = (w_a[..., None] * o_a + w_b[..., None] * o_b) / denom[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, NEG_INF, m_safe + np.log(denom))
    return o, lse


def merge_many(os, lses):
    """Fold a list of partial states with ``merge_states``, left to right."""
    o, lse = os[0], lses[0]
    for o_c, lse_c in zip(os[1:], lses[1:]):
        o, lse = merge_states(o, lse, o_c, lse_c)
    return np.asarray(o, dtype=np.float64), np.asarray(lse, dtype=np.float64)


def attention_rows(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_page_indices,
                   kv_last_page_len, num_qo_heads, num_kv_heads, page_size, causal,
                   window_left, sm_scale, b, rows, heads, kv_begin=None, kv_end=None,
                   custom_mask=None, mask_indptr=None, logits_soft_cap=0.0):
    """``attention`` restricted to some rows and q heads of request b.

    Same definition, float64, for a subset of the outputs (pinned against
    ``attention`` on every row).  rows are request-local query indices, heads
    q-head indices.
    Returns o [len(rows), len(heads), D] and lse [len(rows), len(heads)].
    The request's keys are read page by page through its page table.
    """
    _check_heads(num_qo_heads, num_kv_heads)
    use_custom = _check_custom(custom_mask, mask_indptr, causal)
    group = num_qo_heads // num_kv_heads
    L = int(kv_lengths(kv_indptr, kv_last_page_len, page_size)[b])
    q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
    qo_len = q1 - q0
    first, n_pages = int(kv_indptr[b]), int(kv_indptr[b + 1]) - int(kv_indptr[b])
    pages = np.asarray(kv_page_indices[first:first + n_pages], dtype=np.int64)
    mask = allowed_mask(qo_len, L, causal, window_left, kv_begin, kv_end)
    if use_custom:
        mask = mask & custom_mask_rows(custom_mask, mask_indptr, b, qo_len, L)
    d = np.shape(q)[2]
    o = np.zeros((len(rows), len(heads), d), dtype=np.float64)
    lse = np.full((len(rows), len(heads)), NEG_INF, dtype=np.float64)
    for hi_, h in enumerate(heads):
        g = h // group
        kb = np.asarray(k_pool[pages, :, g, :], dtype=np.float64).reshape(-1, d)[:L]
        vb = np.asarray(v_pool[pages, :, g, :], dtype=np.float64).reshape(-1, d)[:L]
        for ri, i in enumerate(rows):
            ok = mask[i]
            if not ok.any():
                continue
            s = soft_cap(sm_scale * (kb[ok] @ np.asarray(q[q0 + i, h, :], dtype=np.float64)),
                         logits_soft_cap)
            m = s.max()
            e = np.exp(s - m)
            total = e.sum()
            lse[ri, hi_] = m + np.log(total)
            o[ri, hi_] = (e / total) @ vb[ok]
    return o, lse


def append_paged_kv(k_pool, v_pool, append_k, append_v, batch_indices, positions,
                    kv_indptr, kv_page_indices, page_size):
    """Write new key/value rows into a paged cache, returning updated copies.

    Token t belongs to request batch_indices[t] at logical position
    positions[t]; it lands on page kv_page_indices[kv_indptr[b] + pos // P],
    slot pos % P (the same page table attention reads; PR #399, per-commit
    messages, the torch.compile aliasing commit: an append writes scattered
    pages).  Rows are copied exactly; every other slot
    is left untouched.  append_k / append_v: [tokens, Hkv, D].
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for t in range(len(batch_indices)):
        b, pos = int(batch_indices[t]), int(positions[t])
        page = int(kv_page_indices[int(kv_indptr[b]) + pos // page_size])
        k_out[page, pos % page_size] = append_k[t]
        v_out[page, pos % page_size] = append_v[t]
    return k_out, v_out
