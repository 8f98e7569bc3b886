"""ctypes binding of the CPU oracle (test infrastructure only).

Arguments are numpy arrays or CPU torch tensors; bf16 tensors are passed as
their uint16 bit patterns. Results come back as numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import numpy as np

from .build import LIB, build

_lib = None


class OracleShape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_q", C.c_int32), ("d_c", C.c_int32),
                ("num_heads", C.c_int32), ("head_dim", C.c_int32),
                ("block_size", C.c_int32), ("max_pages", C.c_int32),
                ("num_idx_heads", C.c_int32)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        P = C.c_void_p
        sp = C.POINTER(OracleShape)
        L.oracle_set_threads.argtypes = [C.c_int]
        L.oracle_get_threads.argtypes = []
        L.oracle_index_scores.argtypes = [sp, P, P, P, P, P, P, C.c_int64]
        L.oracle_topk_select.argtypes = [sp, P, C.c_int64, P, P, C.c_int32, C.c_int32,
                                         P, P, P, P, P]
        L.oracle_attend.argtypes = [sp, P, P, P, P, P, C.c_int32, C.c_double, P, P, P]
        L.oracle_dense_causal_attention.argtypes = [sp, P, P, P, P, P, P, C.c_double, P, P]
        L.oracle_to_bf16.argtypes = [P, P, C.c_int64]
        L.oracle_mxfp4_to_fp8.argtypes = [P, P, C.c_int64, C.c_int64, C.c_int32, P]
        L.oracle_mxfp4_to_fp8_experts.argtypes = [P, P, C.c_int32, C.c_int64, C.c_int64, P,
                                                  C.c_int32, C.c_int32, P]
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    if lib().oracle_set_threads(int(n)) != 0:
        raise ValueError("thread count must be >= 1")


def get_threads() -> int:
    return int(lib().oracle_get_threads())


def _np(x, dtype):
    """numpy view with the given dtype; bf16 torch tensors become uint16."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16)
            x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype != np.dtype(dtype):
        if dtype == np.uint16 and x.dtype == np.int16:
            x = x.view(np.uint16)
        else:
            x = x.astype(dtype)
    return x


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def shape(batch, num_q, d_c, num_heads, head_dim, block_size, max_pages,
          num_idx_heads=1) -> OracleShape:
    return OracleShape(batch, num_q, d_c, num_heads, head_dim, block_size, max_pages,
                       num_idx_heads)


def _hi(sh) -> int:
    return max(1, int(sh.num_idx_heads))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments")


def index_scores(sh, q_comp, k_comp_cache, page_table, seq_lens, q_start, ld=None,
                 fill=np.nan):
    ld = int(ld if ld is not None else sh.max_pages * sh.block_size)
    qc = _np(q_comp, np.uint16)
    kc = _np(k_comp_cache, np.uint16)
    pt = _np(page_table, np.int32)
    sl = None if seq_lens is None else _np(seq_lens, np.int32)
    qs = None if q_start is None else _np(q_start, np.int32)
    out = np.full((sh.batch, sh.num_q) + ((_hi(sh),) if _hi(sh) > 1 else ()) + (ld,), fill,
                  dtype=np.float32)
    _check(lib().oracle_index_scores(C.byref(sh), _ptr(qc), _ptr(kc), _ptr(pt), _ptr(sl),
                                     _ptr(qs), _ptr(out), ld), "index_scores")
    return out


def topk_select(sh, scores, seq_lens, q_start, topk, n_sel_pages=0):
    s = _np(scores, np.float32)
    ld = s.shape[-1]
    sl = None if seq_lens is None else _np(seq_lens, np.int32)
    qs = None if q_start is None else _np(q_start, np.int32)
    rows = (sh.batch, sh.num_q) + ((_hi(sh),) if _hi(sh) > 1 else ())
    idx = np.empty(rows + (topk,), np.int32)
    w = np.empty(rows + (topk,), np.float32)
    cnt = np.empty(rows, np.int32)
    mask = np.empty(rows + (sh.max_pages,), np.uint64)
    pages = np.empty(rows + (max(n_sel_pages, 1),), np.int32)
    _check(lib().oracle_topk_select(C.byref(sh), _ptr(s), ld, _ptr(sl), _ptr(qs), int(topk),
                                    int(n_sel_pages), _ptr(idx), _ptr(w), _ptr(cnt),
                                    _ptr(mask), _ptr(pages) if n_sel_pages > 0 else None),
           "topk_select")
    return {"idx": idx, "w": w, "count": cnt, "page_mask": mask,
            "sel_pages": pages[..., :n_sel_pages] if n_sel_pages > 0 else None}


def attend(sh, q, k_cache, v_cache, page_table, idx, scale=None, want_probs=False):
    scale = 1.0 / math.sqrt(sh.head_dim) if scale is None else float(scale)
    qa = _np(q, np.uint16)
    ka = _np(k_cache, np.uint16)
    va = _np(v_cache, np.uint16)
    pt = _np(page_table, np.int32)
    ix = _np(idx, np.int32)
    topk = ix.shape[-1]
    rows = (sh.batch, sh.num_q, sh.num_heads)
    out = np.empty(rows + (sh.head_dim,), np.float64)
    lse = np.empty(rows, np.float64)
    probs = np.empty(rows + (topk,), np.float64) if want_probs else None
    _check(lib().oracle_attend(C.byref(sh), _ptr(qa), _ptr(ka), _ptr(va), _ptr(pt), _ptr(ix),
                               topk, scale, _ptr(out), _ptr(lse), _ptr(probs)), "attend")
    return (out, lse, probs) if want_probs else (out, lse)


def dense_causal_attention(sh, q, k_cache, v_cache, page_table, seq_lens, q_start, scale=None):
    scale = 1.0 / math.sqrt(sh.head_dim) if scale is None else float(scale)
    qa = _np(q, np.uint16)
    ka = _np(k_cache, np.uint16)
    va = _np(v_cache, np.uint16)
    pt = _np(page_table, np.int32)
    sl = None if seq_lens is None else _np(seq_lens, np.int32)
    qs = None if q_start is None else _np(q_start, np.int32)
    rows = (sh.batch, sh.num_q, sh.num_heads)
    out = np.empty(rows + (sh.head_dim,), np.float64)
    lse = np.empty(rows, np.float64)
    _check(lib().oracle_dense_causal_attention(C.byref(sh), _ptr(qa), _ptr(ka), _ptr(va),
                                               _ptr(pt), _ptr(sl), _ptr(qs), scale,
                                               _ptr(out), _ptr(lse)), "dense_causal_attention")
    return out, lse


def to_bf16(x):
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    _check(lib().oracle_to_bf16(_ptr(a), _ptr(out), a.size), "to_bf16")
    return out


def mxfp4_to_fp8(packed, scales, rows, cols, exp_offset=0):
    """FP8 E4M3 bit patterns [rows, cols] of one MXFP4 matrix (see oracle.h)."""
    pk = _np(packed, np.uint8)
    sc = _np(scales, np.uint8)
    if pk.size < rows * cols // 2 or sc.size < rows * cols // 32:
        raise ValueError("packed or scales smaller than the matrix")
    out = np.empty((rows, cols), np.uint8)
    _check(lib().oracle_mxfp4_to_fp8(_ptr(pk), _ptr(sc), int(rows), int(cols), int(exp_offset),
                                     _ptr(out)), "mxfp4_to_fp8")
    return out


def mxfp4_to_fp8_experts(packed, scales, num_experts, rows, cols, expert_ids, exp_offset=0,
                         out=None):
    """Slots [n_sel, rows, cols] of the selected experts; `out` (uint8, updated
    in place) keeps slots whose id is out of range."""
    pk = _np(packed, np.uint8)
    sc = _np(scales, np.uint8)
    ids = _np(expert_ids, np.int32).reshape(-1)
    if pk.size < num_experts * rows * cols // 2 or sc.size < num_experts * rows * cols // 32:
        raise ValueError("packed or scales smaller than the expert pool")
    if out is None:
        out = np.zeros((ids.size, rows, cols), np.uint8)
    if out.dtype != np.uint8 or not out.flags.c_contiguous or out.size < ids.size * rows * cols:
        raise ValueError("out must be a contiguous uint8 array of n_sel * rows * cols")
    _check(lib().oracle_mxfp4_to_fp8_experts(_ptr(pk), _ptr(sc), int(num_experts), int(rows),
                                             int(cols), _ptr(ids), int(ids.size),
                                             int(exp_offset), _ptr(out)), "mxfp4_to_fp8_experts")
    return out


def bf16_to_f64(u16):
    """uint16 bf16 bit patterns -> float64 (exact)."""
    u = np.ascontiguousarray(u16).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- workloads

def shape_of(w, num_q=None, batch=None):
    cfg = w.config
    return shape(batch if batch is not None else cfg.batch,
                 num_q if num_q is not None else w.num_q, cfg.d_c, cfg.num_heads,
                 cfg.head_dim, cfg.block_size, w.max_pages, getattr(cfg, "num_idx_heads", 1))


def run(w, rows=None, scale=None, want_probs=False):
    """The whole pipeline on a workload: scores, selection, attention.

    rows: optional list of (b, i) query rows to evaluate one by one (each as a
    batch-1, one-row problem over the same caches); None evaluates every row.
    Returns a dict of numpy arrays shaped [R, ...] for the listed rows, or
    [B, S_q, ...] for all rows.
    """
    cfg = w.config
    if rows is None:
        sh = shape_of(w)
        sc = index_scores(sh, w.q_comp, w.k_comp_cache, w.page_table, w.seq_lens, w.q_start)
        sel = topk_select(sh, sc, w.seq_lens, w.q_start, cfg.topk, cfg.n_sel_pages)
        res = attend(sh, w.q, w.k_cache, w.v_cache, w.page_table, sel["idx"], scale, want_probs)
        out = dict(sel, scores=sc, out=res[0], lse=res[1])
        if want_probs:
            out["probs"] = res[2]
        return out
    outs = []
    for (b, i) in rows:
        sh = shape_of(w, num_q=1, batch=1)
        pt = _np(w.page_table, np.int32)[b:b + 1]
        qs = np.array([int(_np(w.q_start, np.int32)[b]) + i], np.int32)
        qc = _np(w.q_comp, np.uint16)[b:b + 1, i:i + 1]
        qq = _np(w.q, np.uint16)[b:b + 1, i:i + 1]
        sc = index_scores(sh, qc, w.k_comp_cache, pt, None, qs)
        sel = topk_select(sh, sc, None, qs, cfg.topk, cfg.n_sel_pages)
        res = attend(sh, qq, w.k_cache, w.v_cache, pt, sel["idx"], scale, want_probs)
        d = dict(sel, scores=sc, out=res[0], lse=res[1])
        if want_probs:
            d["probs"] = res[2]
        outs.append({k: (None if v is None else v[0, 0]) for k, v in d.items()})
    return {k: (None if outs[0][k] is None else np.stack([o[k] for o in outs]))
            for k in outs[0]}
