"""Paged-KV attention prefill for AMD MI355X (gfx950): thin Python binding.

    p = plan(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len,
             num_qo_heads, num_kv_heads, head_dim, page_size, causal,
             window_left=-1, sm_scale=None, dtype=torch.bfloat16)
    o, lse = p.run(q, paged_k, paged_v)
    o, lse = merge_states(o_a, lse_a, o_b, lse_b)

Every step of the computation runs in the HIP library ``libpkv.so`` (C ABI in
include/pkv.h); this module only marshals arguments.  PyTorch supplies device
memory and the current stream.  There is no fallback: without the built
library, or on a machine without a GPU, calls that compute raise.

Semantics (AMD-Ecosystem FlashInfer fork, PR #339 section "Why
window_size_right stays -1"; PR #362 Summary; PR #399 What changed): masked
softmax(sm_scale * Q K^T) V with a bottom-right causal mask, an optional
left-only window (key j kept for row i when j + qo_len + window_left >=
kv_len + i), GQA (q head h reads kv head h // (Hq // Hkv)), natural-log lse.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

__all__ = ["plan", "plan_host", "verify_plan", "workspace_size", "merge_states", "append_kv",
           "chain_speculative_sampling", "chain_speculative_sampling_no_alloc", "Plan",
           "PkvError", "library_path", "load_library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv.so")
_lib = None

PKV_OK, PKV_EINVAL, PKV_ELAYOUT, PKV_EGQA, PKV_EMISMATCH, PKV_ENOTPLANNED, PKV_EHIP, \
    PKV_EWORKSPACE = range(8)
_STATUS_NAMES = ["OK", "EINVAL", "ELAYOUT", "EGQA", "EMISMATCH", "ENOTPLANNED", "EHIP",
                 "EWORKSPACE"]
PKV_FP16, PKV_BF16, PKV_FP32, PKV_FP8_E4M3 = 0, 1, 2, 3


class PkvError(ValueError):
    """A call refused by the library (status and message from pkv_last_error)."""

    def __init__(self, status, message):
        self.status = status
        self.status_name = _STATUS_NAMES[status] if 0 <= status < len(_STATUS_NAMES) else str(status)
        super().__init__(f"[{self.status_name}] {message}")


class _PlanOptions(ctypes.Structure):
    _fields_ = [("num_kv_chunks", ctypes.c_int32), ("kv_begin", ctypes.c_int32),
                ("kv_end", ctypes.c_int32), ("tile", ctypes.c_int32),
                ("split_tiles", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3),
                ("custom_mask", ctypes.c_void_p), ("mask_indptr", ctypes.c_void_p),
                ("logits_soft_cap", ctypes.c_float), ("kv_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("total_q_rows", ctypes.c_int64), ("num_page_indices", ctypes.c_int64),
                ("batch_size", ctypes.c_int32), ("num_work_items", ctypes.c_int32),
                ("num_merge_items", ctypes.c_int32), ("num_partial_slots", ctypes.c_int32),
                ("tile_rows", ctypes.c_int32), ("tile_keys", ctypes.c_int32),
                ("max_page_index", ctypes.c_int32), ("has_device_copy", ctypes.c_int32),
                ("int_ws_bytes", ctypes.c_int64), ("float_ws_bytes", ctypes.c_int64),
                ("total_kv_len", ctypes.c_int64)]


def library_path():
    return _LIB_PATH


def load_library():
    """Load libpkv.so (built in-tree by paged_kv_cache_prefill_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_prefill_amd.build`")
    # resolve every symbol now: a missing kernel stub must fail here, not mid-run
    lib = ctypes.CDLL(_LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_version.restype = ctypes.c_char_p
    lib.pkv_workspace_size.argtypes = [pi32, pi32, pi32, i64, pi32, i32, i32, i32, i32, i32, i32,
                                       i32, ctypes.POINTER(_PlanOptions), ctypes.POINTER(sz),
                                       ctypes.POINTER(sz)]
    lib.pkv_plan.argtypes = [pi32, pi32, pi32, i64, pi32, i32, i32, i32, i32, i32, i32, i32,
                             ctypes.c_float, ctypes.c_int, vp, sz, vp, sz, vp,
                             ctypes.POINTER(_PlanOptions), ctypes.POINTER(vp)]
    lib.pkv_run.argtypes = [vp, vp, i64, i32, i32, i64, i64,
                            vp, i64, i32, i32, i32, i64, i64, i64,
                            vp, i64, i32, i32, i32, i64, i64, i64,
                            ctypes.c_int, vp, i64, vp, i64, vp]
    lib.pkv_merge_states.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, ctypes.c_int, vp]
    lib.pkv_debug_gather.argtypes = [vp, vp, i64, i32, i32, i32, i64, i64, i64,
                                     vp, i64, i32, i32, i32, i64, i64, i64,
                                     ctypes.c_int, vp, vp, i64, vp]
    lib.pkv_append_kv.argtypes = [vp, i64, i64, vp, i64, i64, i64, i32, i32,
                                  vp, vp, vp, i32, vp, i64,
                                  vp, i64, i32, i64, i64, i64,
                                  vp, i64, i32, i64, i64, i64,
                                  ctypes.c_int, vp, vp]
    lib.pkv_chain_speculative_sampling.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp,
                                                   vp, sz, vp]
    lib.pkv_chain_speculative_sampling_no_alloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32,
                                                            vp, vp, vp]
    lib.pkv_chain_speculative_sampling_workspace_size.argtypes = [i32, i32]
    lib.pkv_chain_speculative_sampling_workspace_size.restype = sz
    lib.pkv_plan_get_info.argtypes = [vp, ctypes.POINTER(_PlanInfo)]
    lib.pkv_plan_get_work.argtypes = [vp, pi32, i64, ctypes.POINTER(i64)]
    lib.pkv_plan_destroy.argtypes = [vp]
    lib.pkv_plan_destroy.restype = None
    for name in ("pkv_workspace_size", "pkv_plan", "pkv_run", "pkv_merge_states",
                 "pkv_debug_gather", "pkv_append_kv", "pkv_chain_speculative_sampling",
                 "pkv_chain_speculative_sampling_no_alloc", "pkv_plan_get_info",
                 "pkv_plan_get_work"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status):
    if status != PKV_OK:
        msg = _lib.pkv_last_error().decode(errors="replace")
        if status == PKV_EHIP:
            raise RuntimeError(f"[EHIP] {msg}")
        raise PkvError(status, msg)


def _torch():
    import torch
    return torch


def _dtype_code(dtype):
    torch = _torch()
    if dtype in (torch.bfloat16, "bf16", "bfloat16"):
        return PKV_BF16
    if dtype in (torch.float16, "fp16", "float16"):
        return PKV_FP16
    if dtype in (torch.float32, "fp32", "float32"):
        return PKV_FP32
    raise PkvError(PKV_EINVAL, f"dtype: expected fp16 or bf16, given {dtype}")


def _host_i32(x, name):
    if x is None:
        return None
    if isinstance(x, np.ndarray) and x.dtype == np.int32 and x.ndim == 1 and \
            x.flags.c_contiguous:
        return x
    if hasattr(x, "detach"):  # torch tensor
        if x.is_cuda:
            raise PkvError(PKV_EINVAL, f"{name}: expected a host array, given a device tensor")
        x = x.detach().numpy()
    a = np.ascontiguousarray(np.asarray(x), dtype=np.int64)
    if a.ndim != 1:
        raise PkvError(PKV_EINVAL, f"{name}: expected a 1-D array, given shape {a.shape}")
    if a.size and (a.min() < -(2 ** 31) or a.max() >= 2 ** 31):
        raise PkvError(PKV_EINVAL, f"{name}: values must fit in int32")
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr_i32(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if a is not None and a.size else None


def _options(num_kv_chunks=0, kv_begin=0, kv_end=-1, tile=0, custom_mask=None,
             mask_indptr=None, logits_soft_cap=0.0, kv_dtype=None, k_scale=1.0, v_scale=1.0,
             split_tiles=0, batch=None):
    o = _PlanOptions()
    o.num_kv_chunks, o.kv_begin, o.kv_end, o.tile = int(num_kv_chunks), int(kv_begin), \
        int(kv_end), int(tile)
    o.split_tiles = int(split_tiles)
    o.logits_soft_cap = float(logits_soft_cap or 0.0)
    if kv_dtype is not None:
        if kv_dtype not in ("fp8_e4m3", PKV_FP8_E4M3) and str(kv_dtype) != "torch.float8_e4m3fn":
            raise PkvError(PKV_EINVAL, f"kv_dtype: expected None or 'fp8_e4m3', given {kv_dtype!r}")
        o.kv_dtype = PKV_FP8_E4M3
        o.k_scale, o.v_scale = float(k_scale), float(v_scale)
    if custom_mask is not None or mask_indptr is not None:
        if custom_mask is None or mask_indptr is None:
            raise PkvError(PKV_EINVAL, "custom_mask and mask_indptr: expected both or neither")
        m = np.ascontiguousarray(np.asarray(custom_mask).reshape(-1), dtype=np.uint8)
        ind = np.ascontiguousarray(np.asarray(mask_indptr).reshape(-1), dtype=np.int64)
        if batch is not None:
            # the library reads mask_indptr[0..batch] and custom_mask[0, mask_indptr[batch])
            if len(ind) != batch + 1:
                raise PkvError(PKV_EINVAL, f"mask_indptr: expected {batch + 1} entries, "
                                           f"given {len(ind)}")
            if int(ind[-1]) > m.size:
                raise PkvError(PKV_EINVAL, f"custom_mask: expected at least mask_indptr[{batch}]"
                                           f" = {int(ind[-1])} bytes, given {m.size}")
        if m.size == 0:
            # a mask of no bytes (every request has no row or no key) still
            # names its storage: NULL would mean "no mask"
            m = np.zeros(1, dtype=np.uint8)
        o.custom_mask = m.ctypes.data
        o.mask_indptr = ind.ctypes.data
        o._keep = (m, ind)   # the arrays must outlive the call
    return o


def _plan_arrays(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len):
    qo = _host_i32(qo_indptr, "qo_indptr")
    kv = _host_i32(kv_indptr, "kv_indptr")
    idx = _host_i32(kv_page_indices, "kv_page_indices")
    last = _host_i32(kv_last_page_len, "kv_last_page_len")
    batch = len(qo) - 1
    if batch < 0 or len(kv) != batch + 1 or len(last) != batch:
        raise PkvError(PKV_EINVAL, f"qo_indptr / kv_indptr / kv_last_page_len: expected lengths "
                                   f"B+1, B+1, B; given {len(qo)}, {len(kv)}, {len(last)}")
    if idx is None:
        idx = np.zeros(0, dtype=np.int32)
    return qo, kv, idx, last, batch


def workspace_size(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
                   num_kv_heads, head_dim, page_size, causal, window_left=-1, sm_scale=None,
                   **opts):
    """(int workspace bytes, float workspace bytes) a plan with these arguments needs."""
    lib = load_library()
    qo, kv, idx, last, batch = _plan_arrays(qo_indptr, kv_indptr, kv_page_indices,
                                            kv_last_page_len)
    ib, fb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    o = _options(**opts)
    _check(lib.pkv_workspace_size(_ptr_i32(qo), _ptr_i32(kv), _ptr_i32(idx), len(idx),
                                  _ptr_i32(last), batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                  int(bool(causal)), int(window_left), ctypes.byref(o),
                                  ctypes.byref(ib), ctypes.byref(fb)))
    return ib.value, fb.value


class Plan:
    """A validated, scheduled batch.  Owns its device workspaces."""

    def __init__(self, handle, dtype, head_dim, num_qo_heads, num_kv_heads, page_size, device,
                 int_ws, float_ws):
        self._h = ctypes.c_void_p(handle)
        self.dtype = dtype
        self.head_dim = head_dim
        self.num_qo_heads = num_qo_heads
        self.num_kv_heads = num_kv_heads
        self.page_size = page_size
        self.device = device
        self._int_ws = int_ws
        self._float_ws = float_ws
        self.kv_fp8 = False
        info = _PlanInfo()
        _check(_lib.pkv_plan_get_info(self._h, ctypes.byref(info)))
        self.info = {name: getattr(info, name) for name, _ in _PlanInfo._fields_}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.pkv_plan_destroy(h)
            self._h = None

    @property
    def total_q_rows(self):
        return self.info["total_q_rows"]

    def work_items(self):
        """Task list as an int32 array [n, 8]:
        (request, kv_head, row0, num_rows, kv_begin, kv_end, partial_slot, tile_begin)."""
        n = ctypes.c_int64(0)
        _check(_lib.pkv_plan_get_work(self._h, None, 0, ctypes.byref(n)))
        out = np.zeros((n.value, 8), dtype=np.int32)
        if n.value:
            _check(_lib.pkv_plan_get_work(self._h, _ptr_i32(out.reshape(-1)), n.value,
                                          ctypes.byref(n)))
        return out

    @staticmethod
    def _cache_view(x, kv_layout):
        if x.dim() != 4:
            raise PkvError(PKV_ELAYOUT, f"paged cache: expected 4-D, given {x.dim()}-D")
        if kv_layout == "HND":      # [pages, heads, page_size, dim] -> logical NHD
            x = x.permute(0, 2, 1, 3)
        elif kv_layout != "NHD":
            raise PkvError(PKV_EINVAL, f"kv_layout: expected 'NHD' or 'HND', given {kv_layout!r}")
        if x.stride(3) != 1:
            raise PkvError(PKV_ELAYOUT, f"paged cache: head_dim stride must be 1, given "
                                        f"{x.stride(3)}")
        return x

    def _stream(self, stream):
        torch = _torch()
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(stream.cuda_stream)

    def run(self, q, paged_k, paged_v, out=None, lse=None, return_lse=True, kv_layout="NHD",
            stream=None):
        """Attention over the planned batch -> (o, lse or None)."""
        torch = _torch()
        if self._int_ws is None:
            raise PkvError(PKV_ENOTPLANNED, "plan was built host-only; it cannot run")
        if q.dim() != 3:
            raise PkvError(PKV_ELAYOUT, f"q: expected [rows, heads, head_dim], given {q.dim()}-D")
        if q.numel() == 0:
            # no query row: strides mean nothing (numpy gives empty arrays zero
            # strides); hand the library packed ones
            q_s_tok, q_s_head = q.shape[1] * q.shape[2], q.shape[2]
        elif q.stride(2) != 1:
            raise PkvError(PKV_ELAYOUT, f"q: head_dim stride must be 1, given {q.stride(2)}")
        else:
            q_s_tok, q_s_head = q.stride(0), q.stride(1)
        kv_ok = (torch.uint8, torch.float8_e4m3fn) if self.kv_fp8 else (self.dtype,)
        for name, t, ok in (("q", q, (self.dtype,)), ("paged_k", paged_k, kv_ok),
                            ("paged_v", paged_v, kv_ok)):
            if t.dtype not in ok:
                raise PkvError(PKV_EMISMATCH, f"{name} dtype: planned {ok[0]}, given {t.dtype}")
            if t.device != self.device:
                raise PkvError(PKV_EMISMATCH, f"{name} device: planned {self.device}, given {t.device}")
        k = self._cache_view(paged_k, kv_layout)
        v = self._cache_view(paged_v, kv_layout)
        rows = self.total_q_rows
        if out is None:
            out = torch.empty((rows, self.num_qo_heads, self.head_dim), dtype=self.dtype,
                              device=self.device)
        elif (out.dtype != self.dtype or out.dim() != 3 or not out.is_contiguous()
              or tuple(out.shape[1:]) != (self.num_qo_heads, self.head_dim)):
            raise PkvError(PKV_ELAYOUT, "out: expected a packed [rows, num_qo_heads, head_dim] "
                                        "tensor of the plan's dtype")
        if lse is None and return_lse:
            lse = torch.empty((rows, self.num_qo_heads), dtype=torch.float32, device=self.device)
        elif lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                                  or lse.dim() != 2 or lse.shape[1] != self.num_qo_heads):
            raise PkvError(PKV_ELAYOUT, "lse: expected a packed fp32 [rows, num_qo_heads] tensor")
        code = _dtype_code(self.dtype)
        _check(_lib.pkv_run(
            self._h, q.data_ptr(), q.shape[0], q.shape[1], q.shape[2], q_s_tok, q_s_head,
            k.data_ptr(), k.shape[0], k.shape[1], k.shape[2], k.shape[3],
            k.stride(0), k.stride(1), k.stride(2),
            v.data_ptr(), v.shape[0], v.shape[1], v.shape[2], v.shape[3],
            v.stride(0), v.stride(1), v.stride(2),
            code, out.data_ptr(), out.shape[0], lse.data_ptr() if lse is not None else None,
            lse.shape[0] if lse is not None else 0, self._stream(stream)))
        return out, lse

    def debug_gather(self, paged_k, paged_v, kv_layout="NHD", k_out=None, v_out=None,
                     stream=None):
        """The attention kernel's own page gathering: logical K and V rows
        [sum kv_len, Hkv, D] as the kernel loads them for this plan (FP8 caches:
        decoded codes in the plan's dtype).  Keys no task of the plan loads are
        left as they are in k_out / v_out (allocated uninitialised if None)."""
        torch = _torch()
        k = self._cache_view(paged_k, kv_layout)
        v = self._cache_view(paged_v, kv_layout)
        total = int(self.info["total_kv_len"])
        shape = (total, self.num_kv_heads, self.head_dim)
        if k_out is None:
            k_out = torch.empty(shape, dtype=self.dtype, device=self.device)
        if v_out is None:
            v_out = torch.empty(shape, dtype=self.dtype, device=self.device)
        for name, t in (("k_out", k_out), ("v_out", v_out)):
            if t.dtype != self.dtype or not t.is_contiguous() or t.dim() != 3 or \
                    tuple(t.shape[1:]) != shape[1:]:
                raise PkvError(PKV_ELAYOUT, f"{name}: expected a packed [rows, "
                                            f"{shape[1]}, {shape[2]}] {self.dtype} tensor")
        _check(_lib.pkv_debug_gather(
            self._h, k.data_ptr(), k.shape[0], k.shape[1], k.shape[2], k.shape[3],
            k.stride(0), k.stride(1), k.stride(2),
            v.data_ptr(), v.shape[0], v.shape[1], v.shape[2], v.shape[3],
            v.stride(0), v.stride(1), v.stride(2),
            _dtype_code(self.dtype), k_out.data_ptr(), v_out.data_ptr(),
            min(k_out.shape[0], v_out.shape[0]), self._stream(stream)))
        return k_out, v_out


def _make_plan(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
               num_kv_heads, head_dim, page_size, causal, window_left, sm_scale, dtype, device,
               host_only, stream, opts):
    lib = load_library()
    qo, kv, idx, last, batch = _plan_arrays(qo_indptr, kv_indptr, kv_page_indices,
                                            kv_last_page_len)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    code = _dtype_code(dtype)
    o = _options(**opts, batch=batch)
    args = (_ptr_i32(qo), _ptr_i32(kv), _ptr_i32(idx), len(idx), _ptr_i32(last), batch,
            int(num_qo_heads), int(num_kv_heads), int(head_dim), int(page_size),
            int(bool(causal)), int(window_left))
    handle = ctypes.c_void_p()
    int_ws = float_ws = None
    torch = _torch()
    tdtype = {PKV_BF16: torch.bfloat16, PKV_FP16: torch.float16}.get(code)
    if host_only:
        _check(lib.pkv_plan(*args, ctypes.c_float(sm_scale), code, None, 0, None, 0, None,
                            ctypes.byref(o), ctypes.byref(handle)))
        dev = None
    else:
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        ib, fb = ctypes.c_size_t(0), ctypes.c_size_t(0)
        _check(lib.pkv_workspace_size(*args, ctypes.byref(o), ctypes.byref(ib), ctypes.byref(fb)))
        int_ws = torch.empty(max(ib.value, 256), dtype=torch.uint8, device=dev)
        float_ws = torch.empty(max(fb.value // 4, 64), dtype=torch.float32, device=dev)
        s = stream if stream is not None else torch.cuda.current_stream(dev)
        _check(lib.pkv_plan(*args, ctypes.c_float(sm_scale), code, int_ws.data_ptr(),
                            int_ws.numel(), float_ws.data_ptr(), float_ws.numel() * 4,
                            ctypes.c_void_p(s.cuda_stream), ctypes.byref(o),
                            ctypes.byref(handle)))
    p = Plan(handle.value, tdtype, int(head_dim), int(num_qo_heads), int(num_kv_heads),
             int(page_size), dev, int_ws, float_ws)
    p.kv_fp8 = o.kv_dtype == PKV_FP8_E4M3
    return p


def plan(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads, num_kv_heads,
         head_dim, page_size, causal, window_left=-1, sm_scale=None, dtype="bf16",
         device="cuda", stream=None, num_kv_chunks=0, kv_begin=0, kv_end=-1, tile=0,
         custom_mask=None, mask_indptr=None, logits_soft_cap=0.0, kv_dtype=None, k_scale=1.0,
         v_scale=1.0, split_tiles=0):
    """Validate and schedule a batch; returns a runnable Plan.

    Host int arrays: qo_indptr[B+1], kv_indptr[B+1], kv_page_indices[kv_indptr[B]],
    kv_last_page_len[B].  sm_scale defaults to 1/sqrt(head_dim).
    num_kv_chunks / kv_begin / kv_end / tile / split_tiles: optional scheduling knobs (see
    include/pkv.h).
    custom_mask (packed uint8 bits) / mask_indptr (int64 byte offsets [B+1]): a
    per-request topology mask for tree drafts, with causal=False (see include/pkv.h).
    logits_soft_cap > 0 caps every scaled logit s to cap * tanh(s / cap).
    kv_dtype="fp8_e4m3": K/V caches hold E4M3 codes (uint8 or torch.float8_e4m3fn),
    values code * k_scale and code * v_scale; q and o keep `dtype`.
    """
    return _make_plan(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
                      num_kv_heads, head_dim, page_size, causal, window_left, sm_scale, dtype,
                      device, False, stream,
                      dict(num_kv_chunks=num_kv_chunks, kv_begin=kv_begin, kv_end=kv_end,
                           tile=tile, custom_mask=custom_mask, mask_indptr=mask_indptr,
                           logits_soft_cap=logits_soft_cap, kv_dtype=kv_dtype, k_scale=k_scale,
                           v_scale=v_scale, split_tiles=split_tiles))


def plan_host(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
              num_kv_heads, head_dim, page_size, causal, window_left=-1, sm_scale=None,
              dtype="bf16", num_kv_chunks=0, kv_begin=0, kv_end=-1, tile=0,
              custom_mask=None, mask_indptr=None, logits_soft_cap=0.0, kv_dtype=None,
              k_scale=1.0, v_scale=1.0, split_tiles=0):
    """Validate and schedule without a device: an inspectable, non-runnable Plan."""
    return _make_plan(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads,
                      num_kv_heads, head_dim, page_size, causal, window_left, sm_scale, dtype,
                      None, True, None,
                      dict(num_kv_chunks=num_kv_chunks, kv_begin=kv_begin, kv_end=kv_end,
                           tile=tile, custom_mask=custom_mask, mask_indptr=mask_indptr,
                           logits_soft_cap=logits_soft_cap, kv_dtype=kv_dtype, k_scale=k_scale,
                           v_scale=v_scale, split_tiles=split_tiles))


def verify_plan(kv_indptr, kv_page_indices, kv_last_page_len, q_len_per_req, num_qo_heads,
                num_kv_heads, head_dim, page_size, sm_scale=None, dtype="bf16", device="cuda",
                **opts):
    """Chain speculative-decode verify: a causal prefill with q_len_per_req rows per request
    (PR #362: qo_indptr advances by the draft length, the mask is bottom-right causal)."""
    batch = len(_host_i32(kv_indptr, "kv_indptr")) - 1
    qo = np.arange(batch + 1, dtype=np.int64) * int(q_len_per_req)
    return plan(qo, kv_indptr, kv_page_indices, kv_last_page_len, num_qo_heads, num_kv_heads,
                head_dim, page_size, True, -1, sm_scale, dtype, device, **opts)


def merge_states(o_a, lse_a, o_b, lse_b, out=None, lse_out=None, stream=None):
    """Combine two partial states over disjoint key sets -> (o, lse).

    o_*: packed [rows, heads, head_dim] fp16/bf16/fp32; lse_*: packed fp32 [rows, heads].
    out / lse_out may be o_a / lse_a for an in-place merge."""
    torch = _torch()
    lib = load_library()
    if o_a.shape != o_b.shape or o_a.dtype != o_b.dtype or o_a.dim() != 3:
        raise PkvError(PKV_EMISMATCH, f"o_a / o_b: expected equal [rows, heads, dim] shapes and "
                                      f"dtypes, given {tuple(o_a.shape)} {o_a.dtype} and "
                                      f"{tuple(o_b.shape)} {o_b.dtype}")
    rows, heads, dim = o_a.shape
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b)):
        if t.dtype != torch.float32 or tuple(t.shape) != (rows, heads):
            raise PkvError(PKV_EMISMATCH, f"{name}: expected fp32 [{rows}, {heads}], given "
                                          f"{t.dtype} {tuple(t.shape)}")
    for name, t in (("o_a", o_a), ("o_b", o_b), ("lse_a", lse_a), ("lse_b", lse_b)):
        if not t.is_contiguous():
            raise PkvError(PKV_ELAYOUT, f"{name}: expected a packed tensor")
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    if out.shape != o_a.shape or out.dtype != o_a.dtype or not out.is_contiguous():
        raise PkvError(PKV_ELAYOUT, "out: expected a packed tensor shaped like o_a")
    if tuple(lse_out.shape) != (rows, heads) or not lse_out.is_contiguous():
        raise PkvError(PKV_ELAYOUT, "lse_out: expected a packed fp32 [rows, heads] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(o_a.device)
    _check(lib.pkv_merge_states(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(),
                                lse_b.data_ptr(), out.data_ptr(), lse_out.data_ptr(), rows,
                                heads, dim, _dtype_code(o_a.dtype),
                                ctypes.c_void_p(stream.cuda_stream)))
    return out, lse_out


def append_kv(append_k, append_v, batch_indices, positions, kv_indptr, kv_page_indices,
              paged_k, paged_v, kv_layout="NHD", err_count=None, stream=None):
    """Write new K/V rows into their pages (in place) and return (paged_k, paged_v).

    append_k / append_v: [tokens, num_kv_heads, head_dim] in the cache's dtype, head_dim
    packed.  batch_indices, positions [tokens], kv_indptr [batch + 1], kv_page_indices:
    int32 tensors on the cache's device.  Token t goes to page
    kv_page_indices[kv_indptr[b] + pos // page_size], slot pos % page_size.  err_count
    (optional int32 device tensor of one element) counts tokens skipped as out of range."""
    torch = _torch()
    lib = load_library()
    k = Plan._cache_view(paged_k, kv_layout)
    v = Plan._cache_view(paged_v, kv_layout)
    dev = paged_k.device
    if paged_v.device != dev or paged_k.dtype != paged_v.dtype:
        raise PkvError(PKV_EMISMATCH, "paged_k / paged_v: expected one device and dtype")
    for name, t in (("append_k", append_k), ("append_v", append_v)):
        if t.dim() != 3 or t.dtype != paged_k.dtype or t.device != dev:
            raise PkvError(PKV_EMISMATCH, f"{name}: expected a [tokens, heads, head_dim] "
                                          f"{paged_k.dtype} tensor on {dev}")
        if t.numel() and t.stride(2) != 1:   # empty tensors may carry any strides
            raise PkvError(PKV_ELAYOUT, f"{name}: head_dim stride must be 1")
        if tuple(t.shape) != (append_k.shape[0], k.shape[2], k.shape[3]):
            raise PkvError(PKV_EMISMATCH, f"{name}: expected [{append_k.shape[0]}, "
                                          f"{k.shape[2]}, {k.shape[3]}], given {tuple(t.shape)}")
    tokens = append_k.shape[0]
    for name, t, n in (("batch_indices", batch_indices, tokens), ("positions", positions, tokens),
                       ("kv_indptr", kv_indptr, None), ("kv_page_indices", kv_page_indices, None)):
        if t.dtype != torch.int32 or t.device != dev or t.dim() != 1 or not t.is_contiguous():
            raise PkvError(PKV_EINVAL, f"{name}: expected a packed 1-D int32 tensor on {dev}")
        if n is not None and t.shape[0] != n:
            raise PkvError(PKV_EMISMATCH, f"{name}: expected {n} entries, given {t.shape[0]}")
    if kv_indptr.shape[0] < 1:
        raise PkvError(PKV_EINVAL, "kv_indptr: expected batch + 1 >= 1 entries")
    if err_count is not None and (err_count.dtype != torch.int32 or err_count.device != dev
                                  or err_count.numel() < 1):
        raise PkvError(PKV_EINVAL, "err_count: expected an int32 device tensor")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _check(lib.pkv_append_kv(
        append_k.data_ptr(), append_k.stride(0), append_k.stride(1),
        append_v.data_ptr(), append_v.stride(0), append_v.stride(1),
        tokens, k.shape[2], k.shape[3],
        batch_indices.data_ptr(), positions.data_ptr(), kv_indptr.data_ptr(),
        kv_indptr.shape[0] - 1, kv_page_indices.data_ptr(), kv_page_indices.shape[0],
        k.data_ptr(), k.shape[0], k.shape[1], k.stride(0), k.stride(1), k.stride(2),
        v.data_ptr(), v.shape[0], v.shape[1], v.stride(0), v.stride(1), v.stride(2),
        _dtype_code(paged_k.dtype), err_count.data_ptr() if err_count is not None else None,
        ctypes.c_void_p(stream.cuda_stream)))
    return paged_k, paged_v


def _sampling_checks(draft_probs, draft_token_ids, target_probs, accept_u, sample_u):
    torch = _torch()
    if target_probs.dim() != 3:
        raise PkvError(PKV_EINVAL, "target_probs: expected [batch, n + 1, vocab]")
    B, n1, V = target_probs.shape
    n = n1 - 1
    dev = target_probs.device
    want = (("draft_probs", draft_probs, torch.float32, (B, n, V)),
            ("draft_token_ids", draft_token_ids, torch.int32, (B, n)),
            ("target_probs", target_probs, torch.float32, (B, n + 1, V)),
            ("accept_u", accept_u, torch.float32, (B, n)),
            ("sample_u", sample_u, torch.float32, (B,)))
    for name, t, dt, shape in want:
        if t.dtype != dt or tuple(t.shape) != shape or t.device != dev or not t.is_contiguous():
            raise PkvError(PKV_EMISMATCH, f"{name}: expected a packed {dt} tensor {shape} on "
                                          f"{dev}, given {t.dtype} {tuple(t.shape)}")
    return B, n, V, dev


def _sampling_outputs(out, num_accepted, B, n, dev):
    torch = _torch()
    if out is None:
        out = torch.empty((B, n + 1), dtype=torch.int32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    for name, t, shape in (("out", out, (B, n + 1)), ("num_accepted", num_accepted, (B,))):
        if t.dtype != torch.int32 or tuple(t.shape) != shape or t.device != dev or \
                not t.is_contiguous():
            raise PkvError(PKV_EMISMATCH, f"{name}: expected a packed int32 tensor {shape}")
    return out, num_accepted


def chain_speculative_sampling(draft_probs, draft_token_ids, target_probs, accept_u, sample_u,
                               out=None, num_accepted=None, workspace=None, stream=None):
    """Accept/reject each request's draft chain -> (output_token_ids [B, n+1] int32,
    num_accepted [B] int32).

    draft_probs [B, n, V] and target_probs [B, n+1, V] float32, draft_token_ids
    [B, n] int32, accept_u [B, n] and sample_u [B] float32 (uniforms in [0, 1)),
    all packed on one device.  See include/pkv.h for the rule."""
    torch = _torch()
    lib = load_library()
    B, n, V, dev = _sampling_checks(draft_probs, draft_token_ids, target_probs, accept_u,
                                    sample_u)
    out, num_accepted = _sampling_outputs(out, num_accepted, B, n, dev)
    need = lib.pkv_chain_speculative_sampling_workspace_size(B, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _check(lib.pkv_chain_speculative_sampling(
        draft_probs.data_ptr(), draft_token_ids.data_ptr(), target_probs.data_ptr(),
        accept_u.data_ptr(), sample_u.data_ptr(), B, n, V, out.data_ptr(),
        num_accepted.data_ptr(), workspace.data_ptr(), workspace.numel(),
        ctypes.c_void_p(stream.cuda_stream)))
    return out, num_accepted


def chain_speculative_sampling_no_alloc(draft_probs, draft_token_ids, target_probs, accept_u,
                                        sample_u, out, num_accepted, stream=None):
    """chain_speculative_sampling through the library's allocation-free entry point:
    the caller passes the outputs, and the library keeps its tile sums in its own
    per-GPU array (calls on one GPU must be ordered; see include/pkv.h)."""
    torch = _torch()
    lib = load_library()
    B, n, V, dev = _sampling_checks(draft_probs, draft_token_ids, target_probs, accept_u,
                                    sample_u)
    if out is None or num_accepted is None:
        raise PkvError(PKV_EINVAL, "out / num_accepted: expected caller-provided tensors")
    out, num_accepted = _sampling_outputs(out, num_accepted, B, n, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _check(lib.pkv_chain_speculative_sampling_no_alloc(
        draft_probs.data_ptr(), draft_token_ids.data_ptr(), target_probs.data_ptr(),
        accept_u.data_ptr(), sample_u.data_ptr(), B, n, V, out.data_ptr(),
        num_accepted.data_ptr(), ctypes.c_void_p(stream.cuda_stream)))
    return out, num_accepted
