"""Python binding of the C ABI in include/tf.h (argument marshalling only).

Every step of the path runs in the HIP library ``libtf.so`` built from ``csrc/``;
torch supplies device memory and the current stream. There is no fallback: if the
library is missing, importing the calls raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtf.so")

TF_OK, TF_E_INVAL, TF_E_RANGE, TF_E_NOMEM, TF_E_UNSUPPORTED, TF_E_DEVICE = range(6)
TF_LAT_BF16, TF_LAT_FP8E4M3_ROWSCALE = 0, 1
TF_PLAN_ONE_WINDOW_FIRST, TF_PLAN_WINDOWS_FIRST = 0, 1

_c_i32 = ctypes.c_int32
_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class tf_geom(ctypes.Structure):
    _fields_ = [("n_caches", _c_i32), ("page_rows", _c_i32), ("latent_dim", _c_i32), ("rope_dim", _c_i32),
                ("pool_ratio", _c_i32), ("index_dim", _c_i32), ("lat_fmt", _c_i32)]


class tf_budget(ctypes.Structure):
    _fields_ = [("room_bytes", _c_i64), ("window_tokens", _c_i64), ("lookahead_rows", _c_i64),
                ("fixed_bytes_per_stream", _c_i64), ("cache_cap_bytes", _c_i64), ("lanes", _c_i32),
                ("policy", _c_i32)]


class tf_plan(ctypes.Structure):
    _fields_ = [("g", tf_geom),
                ("lat_row_bytes", _c_i64), ("rope_row_bytes", _c_i64), ("pkey_row_bytes", _c_i64),
                ("keys_per_page", _c_i64),
                ("off_latent", _c_i64), ("off_scale", _c_i64), ("off_rope", _c_i64), ("off_pkey", _c_i64),
                ("cache_block_bytes", _c_i64), ("page_bytes", _c_i64),
                ("bytes_per_token", _c_i64), ("bytes_per_token_pages", _c_i64),
                ("window_pages", _c_i64), ("n_windows", _c_i64), ("stream_pages", _c_i64),
                ("total_pages", _c_i64), ("cache_bytes", _c_i64), ("fixed_bytes", _c_i64)]


class tf_kv_view(ctypes.Structure):
    _fields_ = [("pool", _vp), ("pt", _vp), ("pt_stride", _c_i32), ("n_streams", _c_i32), ("n_pages", _c_i32),
                ("cache", _c_i32)]


# name -> (restype, argtypes), in the order of include/tf.h
SIGNATURES = {
    "tf_check_page_table": (_c_i32, [_vp, _c_i32, _c_i32, _c_i32]),
    "tf_kv_pool_plan": (_c_i32, [ctypes.POINTER(tf_geom), ctypes.POINTER(tf_budget), ctypes.POINTER(tf_plan)]),
    "tf_prefill_chunk": (_c_i64, [_c_i64, _c_i64]),
    "tf_latent_write": (_c_i32, [ctypes.POINTER(tf_plan), tf_kv_view, _c_i32, _vp, _vp, _vp, _vp, _vp, _c_i32,
                                 _vp, _vp, _vp, _vp]),
    "tf_latent_write_quantize": (_c_i32, [ctypes.POINTER(tf_plan), tf_kv_view, _c_i32, _vp, _vp, _vp, _vp,
                                          _c_i32, _vp, _vp, _vp, _vp]),
    "tf_indexer_logits": (_c_i32, [ctypes.POINTER(tf_plan), tf_kv_view, _c_i32, _vp, _vp, _vp, _vp, _c_i32, _vp,
                                   _c_i64, _vp, _vp]),
    "tf_topk_blocks": (_c_i32, [_vp, _c_i64, _c_i32, _vp, _c_i32, _vp, _vp, ctypes.c_size_t, _vp]),
    "tf_topk_workspace_bytes": (ctypes.c_size_t, [_c_i32, _c_i64, _c_i32]),
    "tf_sparse_mla_attn": (_c_i32, [ctypes.POINTER(tf_plan), tf_kv_view, _c_i32, _vp, _vp, _vp, _c_i32,
                                    ctypes.c_float, _vp, _c_i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "tf_indexer_topk": (_c_i32, [ctypes.POINTER(tf_plan), tf_kv_view, _c_i32, _vp, _vp, _vp, _vp, _c_i32, _c_i64,
                                 _c_i32, _c_i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "tf_indexer_topk_workspace_bytes": (ctypes.c_size_t, [_c_i32, _c_i64, _c_i32, _c_i32]),
    "tf_indexer_topk_fused": (_c_i32, [ctypes.POINTER(tf_plan), tf_kv_view, _c_i32, _vp, _vp, _vp, _vp, _c_i32,
                                       _c_i64, _c_i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "tf_indexer_topk_fused_workspace_bytes": (ctypes.c_size_t, [_c_i32, _c_i64, _c_i32, _c_i32]),
    "tf_candidate_groups": (_c_i32, [_vp, _c_i64, _c_i32, _vp, _c_i32, _c_i32, _vp, _vp, ctypes.c_size_t, _vp]),
    "tf_candidate_groups_workspace_bytes": (ctypes.c_size_t, [_c_i32, _c_i64, _c_i32, _c_i32]),
    "tf_topk_in_candidates": (_c_i32, [_vp, _c_i64, _c_i32, _vp, _vp, _c_i32, _c_i32, _c_i32, _vp, _vp,
                                       ctypes.c_size_t, _vp]),
    "tf_topk_in_candidates_workspace_bytes": (ctypes.c_size_t, [_c_i32, _c_i64, _c_i32]),
    "tf_sparse_mla_attn_noalloc": (_c_i32, [ctypes.POINTER(tf_plan), tf_kv_view, _c_i32, _vp, _vp, _vp, _c_i32,
                                            ctypes.c_float, _vp, _c_i32, _vp, _vp, _vp]),
    "tf_sparse_mla_attn_noalloc_max_bytes": (ctypes.c_size_t, []),
    "tf_dense_mla_attn": (_c_i32, [ctypes.POINTER(tf_plan), tf_kv_view, _c_i32, _vp, _vp, _vp, _c_i32,
                                   ctypes.c_float, _c_i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "tf_attn_workspace_bytes": (ctypes.c_size_t, [_c_i32, _c_i32, _c_i32]),
    "tf_snapshot_copy": (_c_i32, [ctypes.POINTER(tf_plan), tf_kv_view, tf_kv_view, _c_i32, _vp, _vp, _c_i64, _vp]),
    "tf_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtf.so; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_page_table_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class TFError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"tf status {status}: {msg}")
        self.status = status


def _check(status: int):
    if status != TF_OK:
        raise TFError(status, lib().tf_last_error().decode())


class Launch:
    """A device call whose arguments were marshalled once (pointers, sizes, stream);
    calling it enqueues the same work again, on the stream given when it was made.
    The tensors passed in must outlive it; ``keep`` holds the ones the call itself
    allocated (workspaces)."""
    __slots__ = ("_f", "_a", "keep")

    def __init__(self, name: str, args: tuple, keep=()):
        self._f = getattr(lib(), name)
        self._a = args
        self.keep = keep

    def __call__(self):
        s = self._f(*self._a)
        if s != TF_OK:
            raise TFError(s, lib().tf_last_error().decode())


def _run(name: str, args: tuple, prepare: bool, keep=()):
    if prepare:
        return Launch(name, args, keep)
    _check(getattr(lib(), name)(*args))
    return None


# ------------------------------------------------------------------ host calls
def geom(n_caches=1, index_dim=128, fp8=False, rope_dim=64, page_rows=512, latent_dim=512, pool_ratio=4):
    return tf_geom(n_caches, page_rows, latent_dim, rope_dim, pool_ratio, index_dim,
                   TF_LAT_FP8E4M3_ROWSCALE if fp8 else TF_LAT_BF16)


def kv_pool_plan(g: tf_geom, budget: tf_budget | None = None) -> tf_plan:
    p = tf_plan()
    _check(lib().tf_kv_pool_plan(ctypes.byref(g), ctypes.byref(budget) if budget is not None else None,
                                 ctypes.byref(p)))
    return p


def prefill_chunk(history: int, remaining: int) -> int:
    return int(lib().tf_prefill_chunk(history, remaining))


# ------------------------------------------------------------------ device calls
def _ptr(t):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous and on the GPU"
    return t.data_ptr()


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def check_page_table(pt_host, n_pages: int) -> None:
    """Refuse a host page table [streams, pt_stride] (numpy or CPU tensor, int32) that names a
    page outside [0, n_pages) (entries of -1 mean no page); raises TFError (TF_E_RANGE)."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(pt_host), dtype=np.int32)
    assert a.ndim == 2, "page table must be [streams, pt_stride]"
    _check(lib().tf_check_page_table(a.ctypes.data, a.shape[0], a.shape[1], int(n_pages)))


def view(pool, pt, pt_stride: int, n_pages: int, cache: int = 0, n_streams: int | None = None,
         pt_host=None) -> tf_kv_view:
    """pool: uint8 device tensor of n_pages * page_bytes; pt: int32 [streams, pt_stride] or None
    (then stream b's page i is pool page b * pt_stride + i). pt_host: a host copy of pt, checked
    with tf_check_page_table before the view is made."""
    if pt_host is not None:
        check_page_table(pt_host, n_pages)
    if pt is not None:
        import torch
        assert pt.dtype == torch.int32 and pt.dim() == 2 and pt.shape[1] == pt_stride
        ns = pt.shape[0]
    else:
        ns = max(1, n_pages // pt_stride)
    if n_streams is not None:
        ns = n_streams
    v = tf_kv_view(_ptr(pool), _ptr(pt), pt_stride, ns, n_pages, cache)
    v._keep = (pool, pt)   # the view holds raw pointers: keep the tensors alive while it lives
    return v


def latent_write(plan, dst, row_stream, row_pos, latent, rope, row_scale=None,
                 pkey_stream=None, pkey_idx=None, pkeys=None, stream=None, prepare=False):
    n_rows = 0 if row_stream is None else row_stream.numel()
    n_pk = 0 if pkey_stream is None else pkey_stream.numel()
    return _run("tf_latent_write", (ctypes.byref(plan), dst, n_rows, _ptr(row_stream), _ptr(row_pos), _ptr(latent),
                                    _ptr(row_scale), _ptr(rope), n_pk, _ptr(pkey_stream), _ptr(pkey_idx),
                                    _ptr(pkeys), _stream(stream)), prepare)


def latent_write_quantize(plan, dst, row_stream, row_pos, latent, rope, pkey_stream=None, pkey_idx=None,
                          pkeys=None, stream=None, prepare=False):
    """bf16 latent rows coded as e4m3 with a row scale on the device (fp8 plans only)."""
    n_rows = 0 if row_stream is None else row_stream.numel()
    n_pk = 0 if pkey_stream is None else pkey_stream.numel()
    return _run("tf_latent_write_quantize", (ctypes.byref(plan), dst, n_rows, _ptr(row_stream), _ptr(row_pos),
                                             _ptr(latent), _ptr(rope), n_pk, _ptr(pkey_stream), _ptr(pkey_idx),
                                             _ptr(pkeys), _stream(stream)), prepare)


def indexer_logits(plan, keys, row_stream, row_pos, q, w, logits, n_valid=None, stream=None, prepare=False):
    n_rows, H = w.shape
    return _run("tf_indexer_logits", (ctypes.byref(plan), keys, n_rows, _ptr(row_stream), _ptr(row_pos), _ptr(q),
                                      _ptr(w), H, _ptr(logits), logits.shape[1], _ptr(n_valid), _stream(stream)),
                prepare)


def topk_workspace_bytes(n_rows: int, ld: int, k: int) -> int:
    return int(lib().tf_topk_workspace_bytes(n_rows, ld, k))


def topk_blocks(logits, n_valid, k: int, blocks, ws=None, stream=None, prepare=False):
    n_rows, ld = logits.shape
    need = topk_workspace_bytes(n_rows, ld, k)
    if need and ws is None:
        import torch
        ws = torch.empty(need, dtype=torch.uint8, device=logits.device)
    return _run("tf_topk_blocks", (_ptr(logits), ld, n_rows, _ptr(n_valid), k, _ptr(blocks), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream)), prepare, keep=(ws,))


def indexer_topk_workspace_bytes(n_rows: int, ld: int, k: int, key_block: int) -> int:
    return int(lib().tf_indexer_topk_workspace_bytes(n_rows, ld, k, key_block))


def indexer_topk(plan, keys, row_stream, row_pos, q, w, ld: int, k: int, key_block: int, blocks, n_valid=None,
                 ws=None, stream=None, prepare=False):
    n_rows, H = w.shape
    if ws is None:
        import torch
        ws = torch.empty(max(1, indexer_topk_workspace_bytes(n_rows, ld, k, key_block)), dtype=torch.uint8,
                         device=w.device)
    return _run("tf_indexer_topk", (ctypes.byref(plan), keys, n_rows, _ptr(row_stream), _ptr(row_pos), _ptr(q),
                                    _ptr(w), H, int(ld), int(k), int(key_block), _ptr(blocks), _ptr(n_valid),
                                    _ptr(ws), ws.numel(), _stream(stream)), prepare, keep=(ws,))


def indexer_topk_fused_workspace_bytes(n_rows: int, ld: int, k: int, n_heads: int) -> int:
    return int(lib().tf_indexer_topk_fused_workspace_bytes(n_rows, ld, k, n_heads))


def indexer_topk_fused(plan, keys, row_stream, row_pos, q, w, ld: int, k: int, blocks, n_valid=None, ws=None,
                       stream=None, prepare=False):
    n_rows, H = w.shape
    if ws is None:
        import torch
        ws = torch.empty(max(256, indexer_topk_fused_workspace_bytes(n_rows, ld, k, H)), dtype=torch.uint8,
                         device=w.device)
    return _run("tf_indexer_topk_fused", (ctypes.byref(plan), keys, n_rows, _ptr(row_stream), _ptr(row_pos), _ptr(q),
                                          _ptr(w), H, int(ld), int(k), _ptr(blocks), _ptr(n_valid), _ptr(ws),
                                          ws.numel(), _stream(stream)), prepare, keep=(ws,))


def candidate_groups(logits, n_valid, group: int, n_cand: int, cand, ws=None, stream=None, prepare=False):
    n_rows, ld = logits.shape
    if ws is None:
        import torch
        need = int(lib().tf_candidate_groups_workspace_bytes(n_rows, ld, group, n_cand))
        ws = torch.empty(max(16, need), dtype=torch.uint8, device=logits.device)
    return _run("tf_candidate_groups", (_ptr(logits), ld, n_rows, _ptr(n_valid), int(group), int(n_cand), _ptr(cand),
                                        _ptr(ws), ws.numel(), _stream(stream)), prepare, keep=(ws,))


def topk_in_candidates(logits, n_valid, cand, group: int, k: int, blocks, ws=None, stream=None, prepare=False):
    """Top-k of each row with its keys outside the candidate groups read as -inf."""
    n_rows, ld = logits.shape
    need = int(lib().tf_topk_in_candidates_workspace_bytes(n_rows, ld, k))
    if need and ws is None:
        import torch
        ws = torch.empty(need, dtype=torch.uint8, device=logits.device)
    return _run("tf_topk_in_candidates", (_ptr(logits), ld, n_rows, _ptr(n_valid), _ptr(cand), cand.shape[1],
                                          int(group), int(k), _ptr(blocks), _ptr(ws),
                                          0 if ws is None else ws.numel(), _stream(stream)), prepare, keep=(ws,))


def attn_workspace_bytes(n_rows: int, n_heads: int, k: int) -> int:
    return int(lib().tf_attn_workspace_bytes(n_rows, n_heads, k))


def sparse_mla_attn(plan, kv, row_stream, row_pos, q, softmax_scale: float, blocks, out, lse=None, ws=None,
                    stream=None, prepare=False):
    n_rows, n_heads = q.shape[0], q.shape[1]
    k = blocks.shape[1]
    need = attn_workspace_bytes(n_rows, n_heads, k)
    if need and ws is None:
        import torch
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    return _run("tf_sparse_mla_attn", (ctypes.byref(plan), kv, n_rows, _ptr(row_stream), _ptr(row_pos), _ptr(q),
                                       n_heads, float(softmax_scale), _ptr(blocks), k, _ptr(out), _ptr(lse),
                                       _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
                prepare, keep=(ws,))


def sparse_mla_attn_noalloc(plan, kv, row_stream, row_pos, q, softmax_scale: float, blocks, out, lse=None,
                            stream=None, prepare=False):
    """tf_sparse_mla_attn with the library's fixed scratch in place of a workspace: nothing is allocated."""
    n_rows, n_heads = q.shape[0], q.shape[1]
    return _run("tf_sparse_mla_attn_noalloc", (ctypes.byref(plan), kv, n_rows, _ptr(row_stream), _ptr(row_pos),
                                               _ptr(q), n_heads, float(softmax_scale), _ptr(blocks), blocks.shape[1],
                                               _ptr(out), _ptr(lse), _stream(stream)), prepare)


def sparse_mla_attn_noalloc_max_bytes() -> int:
    return int(lib().tf_sparse_mla_attn_noalloc_max_bytes())


def dense_mla_attn(plan, kv, row_stream, row_pos, q, softmax_scale: float, n_blocks: int, out, lse=None, ws=None,
                   stream=None, prepare=False):
    n_rows, n_heads = q.shape[0], q.shape[1]
    need = attn_workspace_bytes(n_rows, n_heads, n_blocks)
    if need and ws is None:
        import torch
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    return _run("tf_dense_mla_attn", (ctypes.byref(plan), kv, n_rows, _ptr(row_stream), _ptr(row_pos), _ptr(q),
                                      n_heads, float(softmax_scale), int(n_blocks), _ptr(out), _ptr(lse),
                                      _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
                prepare, keep=(ws,))


def snapshot_copy(plan, src, dst, src_stream, dst_stream, at: int, stream=None, prepare=False):
    return _run("tf_snapshot_copy", (ctypes.byref(plan), src, dst, src_stream.numel(), _ptr(src_stream),
                                     _ptr(dst_stream), at, _stream(stream)), prepare)
