"""Workload-level calls of the C ABI: allocate outputs, call the entry points.

Marshalling only: every step runs in libtis's kernels.
"""
from __future__ import annotations

import math

import torch

from . import _lib as T


def shape_of(w, num_q=None, batch=None) -> T.Shape:
    cfg = w.config
    return T.make_shape(batch if batch is not None else cfg.batch,
                        num_q if num_q is not None else w.num_q, cfg.d_c, cfg.num_heads,
                        w.max_pages, w.num_phys_pages, cfg.head_dim, cfg.block_size,
                        cfg.num_idx_heads)


def _sel_rows(w, batch=None):
    """Leading dimensions of per-selection-row outputs: (B, S_q) or, with
    several indexer heads, (B, S_q, Hi)."""
    cfg = w.config
    B = cfg.batch if batch is None else batch
    return (B, w.num_q) + ((cfg.num_idx_heads,) if cfg.num_idx_heads > 1 else ())


def index_score(w, fill=float("nan"), q_start="auto"):
    """q_start="auto" uses the workload's; None puts the last row at seq_lens - 1."""
    sh = shape_of(w)
    cap = w.max_pages * w.config.block_size
    scores = torch.full(_sel_rows(w) + (cap,), fill, dtype=torch.float32, device=w.device)
    qs = w.q_start if q_start == "auto" else q_start
    T.sparse_index_score(sh, w.q_comp, w.k_comp_cache, w.page_table, w.seq_lens, qs, scores)
    return scores


def topk_select(w, scores=None, topk=None, n_sel_pages=None, q_start="auto", workspace=None,
                page_mask=True, weights=True):
    """idx, w, count and (unless page_mask is False) the page bitmask of every
    selection row; with weights False only idx and count are asked for."""
    cfg = w.config
    topk = cfg.topk if topk is None else topk
    n_sel_pages = cfg.n_sel_pages if n_sel_pages is None else n_sel_pages
    sh = shape_of(w)
    rows = _sel_rows(w)
    dev = w.device
    out = {
        "idx": torch.empty(rows + (topk,), dtype=torch.int32, device=dev),
        "w": torch.empty(rows + (topk,), dtype=torch.float32, device=dev) if weights else None,
        "count": torch.empty(rows, dtype=torch.int32, device=dev),
        "page_mask": (torch.empty(rows + (w.max_pages,), dtype=torch.int64, device=dev)
                      if page_mask else None),
    }
    qs = w.q_start if q_start == "auto" else q_start
    T.sparse_topk_select(sh, w.q_comp, w.k_comp_cache, scores, w.page_table, w.seq_lens, qs, topk,
                         n_sel_pages, out["idx"], out["w"], out["count"], out["page_mask"],
                         workspace)
    return out


def gather_attend(w, idx, phase=None, scale=0.0, workspace=None):
    cfg = w.config
    if phase is None:
        phase = T.TIS_PHASE_PREFILL if w.num_q > 1 else T.TIS_PHASE_DECODE
    sh = shape_of(w)
    out = torch.empty((cfg.batch, w.num_q, cfg.num_heads, cfg.head_dim), dtype=torch.bfloat16,
                      device=w.device)
    lse = torch.empty((cfg.batch, w.num_q, cfg.num_heads), dtype=torch.float32, device=w.device)
    T.paged_gather_attend(sh, phase, w.q, w.k_cache, w.v_cache, w.page_table, idx, idx.shape[-1],
                          scale, out, lse, workspace)
    return out, lse


def decode_step(w, topk=None, n_sel_pages=None, scale=0.0, workspace=None, outputs=None):
    cfg = w.config
    topk = cfg.topk if topk is None else topk
    n_sel_pages = cfg.n_sel_pages if n_sel_pages is None else n_sel_pages
    sh = shape_of(w)
    dev = w.device
    if outputs is None:
        outputs = {
            "out": torch.empty((cfg.batch, 1, cfg.num_heads, cfg.head_dim), dtype=torch.bfloat16,
                               device=dev),
            "idx": torch.empty(_sel_rows(w) + (topk,), dtype=torch.int32, device=dev),
            "w": torch.empty(_sel_rows(w) + (topk,), dtype=torch.float32, device=dev),
            "lse": torch.empty((cfg.batch, 1, cfg.num_heads), dtype=torch.float32, device=dev),
        }
    T.sparse_decode_step(sh, w.q_comp, w.k_comp_cache, w.q, w.k_cache, w.v_cache, w.page_table,
                         w.seq_lens, topk, n_sel_pages, scale, outputs["out"], outputs["idx"],
                         outputs["w"], outputs["lse"], workspace)
    return outputs


def append(w, step: int):
    """Append stream step `step`'s rows to w's caches (in place, on the GPU)."""
    st = w.stream
    sh = shape_of(w)
    T.paged_kv_append(sh, st.k_comp_new[step].contiguous(), st.k_new[step].contiguous(),
                      st.v_new[step].contiguous(), w.page_table, w.seq_lens, w.k_comp_cache,
                      w.k_cache, w.v_cache)


def default_scale(w) -> float:
    return 1.0 / math.sqrt(w.config.head_dim)


class Fp8Workspace:
    """One FP8 working buffer reused by every layer's experts ("Day-0
    Adaptation for Trillion-Parameter MoE Models", section V: one reusable FP8
    workspace serves the active experts of the current layer and is then
    handed to the next layer). The buffer is sized once for the largest layer;
    `load` dequantises a layer's selected experts into it and returns the
    [n_sel, rows, cols] view (E4M3 bit patterns), valid until the next load."""

    def __init__(self, max_sel: int, rows: int, cols: int, device="cuda"):
        self.rows, self.cols, self.max_sel = int(rows), int(cols), int(max_sel)
        self.buf = torch.empty(self.max_sel * self.rows * self.cols, dtype=torch.uint8,
                               device=device)

    def load(self, packed, scales, expert_ids, exp_offset=0):
        E = packed.shape[0]
        n = int(expert_ids.numel())
        if n > self.max_sel:
            raise ValueError(f"{n} experts exceed the workspace's {self.max_sel} slots")
        if packed.shape[1] != self.rows or packed.shape[2] * 2 != self.cols:
            raise ValueError("weights do not match the workspace's matrix shape")
        T.mxfp4_to_fp8_experts(packed, scales, E, self.rows, self.cols, expert_ids, self.buf,
                               exp_offset)
        return self.buf[: n * self.rows * self.cols].view(n, self.rows, self.cols)
