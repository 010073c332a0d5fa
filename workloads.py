"""Seeded synthetic inputs for paged-KV attention prefill.

This module only draws inputs: request lengths, a permuted page table, page
pools and queries, with values ~ N(0, 1) rounded to bf16/fp16.  It holds none
of the attention arithmetic and is shared by the tests, the benchmark and the
smoke check, which feed the same arrays to the CPU oracle and to the library.

Recipe (one numpy Generator per workload, seed = 1000 * config + variant):
  1. lengths are drawn first, as inclusive integers;
  2. pages: needed = sum ceil(kv_len / P); the pool holds ceil(1.5 * needed)
     pages; physical ids are a permutation of the pool, handed out in request
     order (or the identity table 0..needed-1 when ``permute`` is False);
  3. q [sum qo_len, Hq, D] and the K and V pools, NHD [pages, P, Hkv, D],
     ~ N(0, 1) in float32, rounded to the storage type (round to nearest even);
  4. with ``poison`` every unreferenced page and every slot past a request's
     last_page_len is NaN, so a stray read shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16, FP16 = "bf16", "fp16"


def round_float32_to_bf16_bits(x):
    """float32 array -> bf16 bit patterns (int16 view), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = bits.astype(np.uint16)
    out[nan] = 0x7FC0
    return out.view(np.int16)


def bf16_bits_to_float32(bits):
    bits = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32)


def draw_values(rng, shape, dtype):
    """N(0, 1) values in the storage type: int16 bf16 bits or float16."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == BF16:
        return round_float32_to_bf16_bits(x)
    if dtype == FP16:
        return x.astype(np.float16)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_float(arr, dtype):
    """Storage array -> exact float32 values."""
    if dtype == BF16:
        return bf16_bits_to_float32(arr)
    return np.asarray(arr, dtype=np.float32)


def nan_value(dtype):
    return np.int16(0x7FC0) if dtype == BF16 else np.float16(np.nan)


@dataclasses.dataclass
class Workload:
    name: str
    qo_lens: np.ndarray
    kv_lens: np.ndarray
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_page_indices: np.ndarray
    kv_last_page_len: np.ndarray
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    causal: bool
    window_left: int
    sm_scale: float
    dtype: str
    q: np.ndarray = None       # storage arrays (int16 bf16 bits or float16)
    k_pool: np.ndarray = None
    v_pool: np.ndarray = None
    custom_mask: np.ndarray = None   # packed topology bits (uint8) and their
    mask_indptr: np.ndarray = None   # per-request byte offsets, or None
    logits_soft_cap: float = 0.0     # 0: no cap

    @property
    def batch_size(self):
        return len(self.qo_lens)

    @property
    def total_q(self):
        return int(self.qo_indptr[-1])

    def plan_args(self):
        return dict(qo_indptr=self.qo_indptr, kv_indptr=self.kv_indptr,
                    kv_page_indices=self.kv_page_indices,
                    kv_last_page_len=self.kv_last_page_len,
                    num_qo_heads=self.num_qo_heads, num_kv_heads=self.num_kv_heads,
                    head_dim=self.head_dim, page_size=self.page_size,
                    causal=self.causal, window_left=self.window_left,
                    sm_scale=self.sm_scale,
                    **({} if self.custom_mask is None else
                       dict(custom_mask=self.custom_mask, mask_indptr=self.mask_indptr)),
                    **({} if not self.logits_soft_cap else
                       dict(logits_soft_cap=self.logits_soft_cap)))

    def float_inputs(self):
        return (to_float(self.q, self.dtype), to_float(self.k_pool, self.dtype),
                to_float(self.v_pool, self.dtype))

    def with_window(self, window_left, causal=None):
        w = dataclasses.replace(self, window_left=int(window_left))
        if causal is not None:
            w.causal = bool(causal)
        return w


def make_page_table(rng, kv_lens, page_size, pool_factor=1.5, permute=True):
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    n_pages = (kv_lens + page_size - 1) // page_size
    needed = int(n_pages.sum())
    num_pages = max(1, int(math.ceil(pool_factor * needed)))
    ids = rng.permutation(num_pages)[:needed] if permute else np.arange(needed)
    kv_indptr = np.zeros(len(kv_lens) + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(n_pages)
    last = np.where(n_pages > 0, kv_lens - (n_pages - 1) * page_size, 0)
    # a request without pages still carries a last_page_len entry; 1 is the
    # neutral value (it is never read because the request has no page)
    last = np.where(n_pages > 0, last, 1)
    return kv_indptr, ids.astype(np.int32), last.astype(np.int32), num_pages


def build(name, qo_lens, kv_lens, num_qo_heads, num_kv_heads, head_dim, page_size,
          causal, window_left, dtype, seed, rng=None, pool_factor=1.5, permute=True,
          poison=False, sm_scale=None, values=True):
    rng = np.random.default_rng(seed) if rng is None else rng
    qo_lens = np.asarray(qo_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    qo_indptr = np.zeros(len(qo_lens) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    kv_indptr, ids, last, num_pages = make_page_table(rng, kv_lens, page_size,
                                                      pool_factor, permute)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    w = Workload(name=name, qo_lens=qo_lens, kv_lens=kv_lens, qo_indptr=qo_indptr,
                 kv_indptr=kv_indptr, kv_page_indices=ids, kv_last_page_len=last,
                 num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, page_size=page_size, num_pages=num_pages,
                 causal=bool(causal), window_left=int(window_left),
                 sm_scale=float(sm_scale), dtype=dtype)
    if values:
        total_q = int(qo_indptr[-1])
        w.q = draw_values(rng, (total_q, num_qo_heads, head_dim), dtype)
        pool_shape = (num_pages, page_size, num_kv_heads, head_dim)
        w.k_pool = draw_values(rng, pool_shape, dtype)
        w.v_pool = draw_values(rng, pool_shape, dtype)
        if poison:
            poison_unreferenced(w)
    return w


def poison_unreferenced(w):
    """NaN into every page no request references and every slot past last."""
    nan = nan_value(w.dtype)
    used = np.zeros(w.num_pages, dtype=bool)
    used[w.kv_page_indices] = True
    for pool in (w.k_pool, w.v_pool):
        pool[~used] = nan
        for b in range(w.batch_size):
            n = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
            if n == 0:
                continue
            last_page = int(w.kv_page_indices[w.kv_indptr[b + 1] - 1])
            pool[last_page, int(w.kv_last_page_len[b]):] = nan


# ----------------------------------------------------------------------------
# The five workloads: shapes, sizes and distributions of the pages' benchmarks.
# ----------------------------------------------------------------------------

def config1(variant=0, window_left=-1, page_size=16, permute=False, **kw):
    """Single request, contiguous KV: qo 16, kv 128, Hq 4 / Hkv 2, D 64, fp16,
    causal.  Contiguous KV is an identity page table (page 16) or one page of 128."""
    return build("single_contiguous", [16], [128], 4, 2, 64, page_size, True,
                 window_left, FP16, seed=1000 * 1 + variant, permute=permute, **kw)


def config2(variant=0, window_left=-1, **kw):
    """Paged batch prefill: batch 8, qo ~ U[128, 1024], kv = qo + U[0, 2048],
    page 16, pool 1.5x, Hq 32 / Hkv 8, D 128, bf16, causal."""
    rng = np.random.default_rng(1000 * 2 + variant)
    qo = rng.integers(128, 1024, size=8, endpoint=True)
    kv = qo + rng.integers(0, 2048, size=8, endpoint=True)
    return build("paged_prefill_b8", qo, kv, 32, 8, 128, 16, True, window_left, BF16,
                 seed=None, rng=rng, **kw)


def config3(variant=0, window_left=0, page_size=16, **kw):
    """Non-causal sliding-window paged prefill: batch 4, qo 512, kv 4096,
    page 1024 or 16, Hq 32 / Hkv 8, D 128, bf16, causal False."""
    return build("noncausal_window_b4", [512] * 4, [4096] * 4, 32, 8, 128, page_size,
                 False, window_left, BF16, seed=1000 * 3 + variant, **kw)


def config4(variant=0, batch=16, num_kv_heads=8, **kw):
    """Speculative-decode verify: 4 chain-draft queries per request,
    kv ~ U[512, 8192], page 16, Hq 32, Hkv 4 or 8, D 128, bf16, causal."""
    rng = np.random.default_rng(1000 * 4 + variant)
    kv = rng.integers(512, 8192, size=batch, endpoint=True)
    return build(f"verify_b{batch}_hkv{num_kv_heads}", [4] * batch, kv, 32,
                 num_kv_heads, 128, 16, True, -1, BF16, seed=None, rng=rng, **kw)


def config5(variant=0, qo_len=64, window_left=-1, **kw):
    """Long-context split-KV: batch 2, qo 1 or 64, kv 65536, page 16,
    Hq 64 / Hkv 8, D 128, bf16, causal; the KV is split into 8 chunks."""
    return build(f"long_ctx_q{qo_len}", [qo_len] * 2, [65536] * 2, 64, 8, 128, 16,
                 True, window_left, BF16, seed=1000 * 5 + variant, **kw)


CONFIG5_CHUNKS = 8


# ----------------------------------------------------------------------------
# Tree drafts: topology masks (input encoding only; no attention arithmetic)
# ----------------------------------------------------------------------------

def pack_custom_mask(mats):
    """Pack per-request boolean [qo_len, kv_len] matrices: row-major bits,
    little-endian within each byte, each request from a fresh byte.
    Returns (uint8 bytes, int64 byte offsets [batch + 1])."""
    segs = [np.packbits(np.asarray(m, dtype=bool).reshape(-1), bitorder="little")
            for m in mats]
    indptr = np.zeros(len(segs) + 1, dtype=np.int64)
    indptr[1:] = np.cumsum([len(x) for x in segs])
    data = np.concatenate(segs) if segs else np.zeros(0, np.uint8)
    return data.astype(np.uint8), indptr


def random_tree_parents(rng, n):
    """Parent of each draft node (-1: a root, hanging off the prefix); nodes are
    numbered so every parent precedes its children."""
    return np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, n)], dtype=np.int64)


def tree_topology_mask(prefix_len, parents):
    """[n, prefix_len + n] mask of a draft tree after a shared prefix: node i
    sees the whole prefix, itself and its ancestors."""
    n = len(parents)
    m = np.zeros((n, prefix_len + n), dtype=bool)
    m[:, :prefix_len] = True
    for i in range(n):
        j = i
        while j >= 0:
            m[i, prefix_len + j] = True
            j = int(parents[j])
    return m


def tree_verify(variant=0, batch=16, num_kv_heads=8, tree_size=8, **kw):
    """Tree-draft verify: per request a random draft tree of tree_size nodes
    after a prefix ~ U[512, 8192], page 16, Hq 32, D 128, bf16, the topology
    as a custom mask (causal off)."""
    rng = np.random.default_rng(1000 * 6 + variant)
    prefix = rng.integers(512, 8192, size=batch, endpoint=True)
    parents = [random_tree_parents(rng, tree_size) for _ in range(batch)]
    w = build(f"tree_verify_b{batch}_hkv{num_kv_heads}", [tree_size] * batch,
              prefix + tree_size, 32, num_kv_heads, 128, 16, False, -1, BF16, seed=None,
              rng=rng, **kw)
    w.custom_mask, w.mask_indptr = pack_custom_mask(
        [tree_topology_mask(int(p), par) for p, par in zip(prefix, parents)])
    return w



# ----------------------------------------------------------------------------
# Chain speculative sampling: draft / target distributions and uniforms
# ----------------------------------------------------------------------------

def _softmax32(logits):
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def spec_sampling_inputs(variant=0, batch=64, num_spec=4, vocab=128256, spread=3.0,
                         draft_noise=1.0):
    """Target probabilities softmax(N(0, spread^2) logits) over the vocabulary at
    num_spec + 1 positions; draft probabilities from the same logits plus
    N(0, draft_noise^2) noise at the first num_spec (a correlated draft model);
    draft tokens drawn from the draft probabilities; accept / sample uniforms
    in [0, 1).  float32 throughout, draft ids int32."""
    rng = np.random.default_rng(1000 * 7 + variant)
    logits = rng.standard_normal((batch, num_spec + 1, vocab), dtype=np.float32) * spread
    target = _softmax32(logits)
    noisy = logits[:, :num_spec] + rng.standard_normal((batch, num_spec, vocab),
                                                       dtype=np.float32) * draft_noise
    draft = _softmax32(noisy)
    cdf = np.cumsum(draft.astype(np.float64), axis=-1)
    u = rng.random((batch, num_spec))
    ids = np.minimum((cdf < (u * cdf[..., -1])[..., None]).sum(axis=-1), vocab - 1)
    return dict(draft_probs=draft, draft_token_ids=ids.astype(np.int32), target_probs=target,
                accept_u=rng.random((batch, num_spec), dtype=np.float32),
                sample_u=rng.random(batch, dtype=np.float32))



# ----------------------------------------------------------------------------
# FP8 E4M3 caches (input encoding only)
# ----------------------------------------------------------------------------

E4M3_NAN = np.uint8(0x7F)


def e4m3_codes(values):
    """Round float32 values to FP8 E4M3 codes (uint8) with torch's encoder."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_pools(w, seed, scale_k=1.0, scale_v=1.0, poison=True):
    """K/V pools of w's shape as E4M3 codes of N(0, 1) / scale (so that code *
    scale is N(0, 1)-like); NaN codes in unreferenced pages and past each
    request's last key when poisoned."""
    rng = np.random.default_rng(seed)
    shape = (w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
    k = e4m3_codes(rng.standard_normal(shape, dtype=np.float32) / np.float32(scale_k))
    v = e4m3_codes(rng.standard_normal(shape, dtype=np.float32) / np.float32(scale_v))
    if poison:
        used = np.zeros(w.num_pages, dtype=bool)
        used[w.kv_page_indices] = True
        for pool in (k, v):
            pool[~used] = E4M3_NAN
            for b in range(w.batch_size):
                if int(w.kv_indptr[b + 1] - w.kv_indptr[b]) == 0:
                    continue
                last_page = int(w.kv_page_indices[w.kv_indptr[b + 1] - 1])
                pool[last_page, int(w.kv_last_page_len[b]):] = E4M3_NAN
    return k, v
