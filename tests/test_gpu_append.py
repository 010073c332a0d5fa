"""Paged-KV append on the GPU against the oracle: every byte of both pools must
match oracle.append_paged_kv (bit-exact copy, untouched slots unchanged), bad
tokens are counted and skipped, and attention over a cache filled by append
equals the oracle's attention over the same logical keys."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (assert_close, device_inputs, oracle_full, plan_for, require_gpu,
                      to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _bits(t):
    """Device fp16/bf16 tensor -> host uint16 array of its bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _host_bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def _case(seed, kv_lens, n_append, heads, dim, page, dtype):
    """Pools with random contents, the page table of kv_lens, and the last
    n_append[b] positions of each request as the tokens to append (the step a
    prefill chunk or a speculative draft performs before attention)."""
    rng = np.random.default_rng(seed)
    kv_indptr, pages, _, num_pages = W.make_page_table(rng, kv_lens, page)
    k_pool = W.draw_values(rng, (num_pages, page, heads, dim), dtype)
    v_pool = W.draw_values(rng, (num_pages, page, heads, dim), dtype)
    bi, pos = [], []
    for b, (L, n) in enumerate(zip(kv_lens, n_append)):
        bi += [b] * n
        pos += list(range(L - n, L))
    order = rng.permutation(len(bi))           # token order must not matter
    bi = np.asarray(bi, np.int32)[order]
    pos = np.asarray(pos, np.int32)[order]
    ak = W.draw_values(rng, (len(bi), heads, dim), dtype)
    av = W.draw_values(rng, (len(bi), heads, dim), dtype)
    return dict(k_pool=k_pool, v_pool=v_pool, ak=ak, av=av, bi=bi, pos=pos,
                kv_indptr=kv_indptr, pages=pages, page=page, dtype=dtype)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _append(pk, c, layout="NHD", err=None):
    k = to_device(c["k_pool"], c["dtype"])
    v = to_device(c["v_pool"], c["dtype"])
    if layout == "HND":
        k = k.permute(0, 2, 1, 3).contiguous()
        v = v.permute(0, 2, 1, 3).contiguous()
    pk.append_kv(to_device(c["ak"], c["dtype"]), to_device(c["av"], c["dtype"]),
                 _i32(c["bi"]), _i32(c["pos"]), _i32(c["kv_indptr"]), _i32(c["pages"]),
                 k, v, kv_layout=layout, err_count=err)
    torch.cuda.synchronize()
    if layout == "HND":
        k = k.permute(0, 2, 1, 3)
        v = v.permute(0, 2, 1, 3)
    return _bits(k), _bits(v)


def _expected(c, valid=None):
    sel = slice(None) if valid is None else valid
    return oracle.append_paged_kv(_host_bits(c["k_pool"]), _host_bits(c["v_pool"]),
                                  _host_bits(c["ak"])[sel], _host_bits(c["av"])[sel],
                                  c["bi"][sel], c["pos"][sel], c["kv_indptr"], c["pages"],
                                  c["page"])


@pytest.mark.parametrize("dtype", [W.FP16, W.BF16])
@pytest.mark.parametrize("page,dim,layout", [(16, 128, "NHD"), (5, 64, "NHD"), (1, 128, "NHD"),
                                             (16, 128, "HND"), (128, 64, "HND")])
def test_append_bit_exact(pk, dtype, page, dim, layout):
    # decode-like (1 token), draft-like (4), chunk-like (37, crossing pages), whole request
    c = _case(11 + page, [40, 9, 300, 37, 1], [1, 4, 37, 37, 1], 4, dim, page, dtype)
    got_k, got_v = _append(pk, c, layout)
    want_k, want_v = _expected(c)
    assert np.array_equal(got_k, want_k)
    assert np.array_equal(got_v, want_v)


def test_append_large_batch_bit_exact(pk):
    # 64 requests x 4 draft tokens, 8 kv heads, head_dim 128, 16-key pages, bf16
    rng = np.random.default_rng(5)
    kv_lens = rng.integers(1024, 8192, size=64)
    c = _case(12, kv_lens, [4] * 64, 8, 128, 16, W.BF16)
    got_k, got_v = _append(pk, c)
    want_k, want_v = _expected(c)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)


def test_append_skips_and_counts_bad_tokens(pk):
    c = _case(13, [40, 20], [5, 3], 2, 64, 16, W.FP16)
    n = len(c["bi"])
    # corrupt four tokens: unknown request (two ways), negative position, and a
    # position past the request's pages; plus a page table entry outside the pool
    bad = np.zeros(n, bool)
    c["bi"][0] = -1
    c["bi"][1] = 7
    c["pos"][2] = -3
    c["pos"][3] = 48          # past the last page of either request (3 and 2 pages of 16)
    bad[:4] = True
    pages = c["pages"].copy()
    num_pages = c["k_pool"].shape[0]
    # the page of request 1 holding position 16 points past the pool
    r1_page1 = int(c["kv_indptr"][1]) + 1
    pages[r1_page1] = num_pages + 2
    c["pages"] = pages
    hits_bad_page = (c["bi"] == 1) & (c["pos"] >= 16) & ~bad
    bad |= hits_bad_page
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got_k, got_v = _append(pk, c, err=err)
    assert int(err.item()) == int(bad.sum())
    want_k, want_v = _expected(c, valid=~bad)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)


def test_append_zero_tokens_is_a_no_op(pk):
    c = _case(14, [10], [0], 2, 64, 16, W.BF16)
    got_k, got_v = _append(pk, c)
    assert np.array_equal(got_k, _host_bits(c["k_pool"]))
    assert np.array_equal(got_v, _host_bits(c["v_pool"]))


@pytest.mark.parametrize("window_left", [-1, 50])
def test_attention_over_appended_cache(pk, window_left):
    """Fill an all-NaN cache through append only, then attend: the result must
    be the oracle's attention over the workload the keys came from."""
    w = W.build("appended", [30, 1, 64], [200, 77, 64], 8, 2, 128, 16, True, window_left,
                W.BF16, seed=15)
    tokens_b, tokens_pos, ks, vs = [], [], [], []
    for b in range(w.batch_size):
        L = int(w.kv_lens[b])
        j = np.arange(L)
        ids = w.kv_page_indices[int(w.kv_indptr[b]) + j // w.page_size]
        kb = w.k_pool[ids, j % w.page_size]          # storage bits, not floats
        vb = w.v_pool[ids, j % w.page_size]
        tokens_b += [b] * L
        tokens_pos += list(range(L))
        ks.append(kb)
        vs.append(vb)
    q, _, _ = device_inputs(w)
    nan = torch.full((w.k_pool.shape[0],) + w.k_pool.shape[1:], float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    k, v = nan.clone(), nan.clone()
    pk.append_kv(to_device(np.concatenate(ks), w.dtype), to_device(np.concatenate(vs), w.dtype),
                 _i32(tokens_b), _i32(tokens_pos), _i32(w.kv_indptr), _i32(w.kv_page_indices),
                 k, v)
    p = plan_for(pk, w)
    o, lse = p.run(q, k, v)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle_full(w)
    assert_close(o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_lse, w.dtype,
                 "attention after append")
