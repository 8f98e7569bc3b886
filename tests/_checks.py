"""Parity checks between the HIP path and the CPU oracle (test helpers).

Acceptance rules:
  * index sets: equal counts; every position in the symmetric difference must
    have an oracle fp32 score within 1e-4 relative of the oracle's K'-th score;
  * selection on identical scores: bit-exact (the oracle's selection run on the
    GPU's own fp32 scores must reproduce the GPU's idx, w, count and mask);
  * attention outputs: |out_gpu - out_oracle| <= 2e-2 + 1e-2 |out_oracle|,
    with out_oracle the oracle's attention over the GPU's own index set;
  * scores: within the fp32 dot-product forward-error bound
    gamma_n * sum_c |q_c k_c| (gamma_n = n u / (1 - n u), u = 2^-24) plus the
    oracle's own final rounding; bit-exact for integer-valued inputs.
"""
from __future__ import annotations

import math
from dataclasses import replace

import numpy as np
import torch

from oracle import oracle as O
from top_index_selection_amd import workloads as W

REL_TIE = 1e-4
ATOL, RTOL = 2e-2, 1e-2
U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def compact(w: W.Workload, b: int, device="cpu") -> W.Workload:
    """Sequence b alone, its pages gathered in logical order (identity table)."""
    cfg = w.config
    bs = cfg.block_size
    n_pages = int((w.page_table[b] >= 0).sum())
    pages = w.page_table[b, :n_pages].long()
    mv = lambda t: t.to(device)
    pt = torch.arange(n_pages, dtype=torch.int32).reshape(1, -1)
    new_cfg = replace(cfg, batch=1, lengths=("list", (int(w.seq_lens[b]),)))
    return W.Workload(new_cfg, w.seed, mv(w.seq_lens[b:b + 1]), mv(w.q_start[b:b + 1]), w.num_q,
                      n_pages, n_pages, mv(pt), mv(w.q_comp[b:b + 1]),
                      mv(w.k_comp_cache[pages]), mv(w.k_cache[pages]), mv(w.v_cache[pages]),
                      mv(w.q[b:b + 1]))


def oracle_scores_row(wc: W.Workload, i: int = 0):
    """Oracle fp32 scores of row i of a batch-1 CPU workload, [p + 1]."""
    sh = O.shape_of(wc, num_q=1, batch=1)
    p = int(wc.q_start[0]) + i
    qs = np.array([p], np.int32)
    sc = O.index_scores(sh, wc.q_comp[:, i:i + 1], wc.k_comp_cache, wc.page_table, None, qs)
    return sc[0, 0, : p + 1]


def abs_dot_bound(wc: W.Workload, i: int = 0):
    """gamma_{d_c} * sum_c |q_c k_c| per position, plus half an ulp for the
    oracle's own rounding of its fp64 sum."""
    p = int(wc.q_start[0]) + i
    k = W.logical_rows(wc.k_comp_cache, wc.page_table, 0, p + 1).to(torch.float64).numpy()
    q = wc.q_comp[0, i].to(torch.float64).numpy()
    s_abs = np.abs(k) @ np.abs(q)
    return gamma(wc.config.d_c) * s_abs


def check_scores(gpu_row, or_row, bound, exact=False):
    gpu_row = np.asarray(gpu_row, np.float64)
    or_row = np.asarray(or_row, np.float64)
    if exact:
        np.testing.assert_array_equal(gpu_row, or_row)
        return 0.0
    err = np.abs(gpu_row - or_row)
    lim = bound + U * np.abs(or_row) + 1e-30
    worst = float((err / lim).max()) if err.size else 0.0
    assert (err <= lim).all(), f"score error beyond the fp32 bound (worst ratio {worst:.3g})"
    return worst


def select_on_scores(scores_row, p, topk, n_sel_pages, block_size=64):
    """The oracle's selection on an explicit fp32 score row (batch 1, 1 row)."""
    ld = (p // block_size + 1) * block_size
    sc = np.zeros((1, 1, ld), np.float32)
    sc[0, 0, : p + 1] = np.asarray(scores_row, np.float32)[: p + 1]
    sh = O.shape(1, 1, 1, 1, 1, block_size, ld // block_size)
    res = O.topk_select(sh, sc, None, np.array([p], np.int32), topk, n_sel_pages)
    return {k: (None if v is None else v[0, 0]) for k, v in res.items()}


def check_selection_exact(gpu, ref, topk, max_pages=None):
    """GPU selection vs the oracle's selection on the same fp32 scores."""
    np.testing.assert_array_equal(np.asarray(gpu["idx"]), ref["idx"])
    k = int(ref["count"])
    if gpu.get("count") is not None:
        assert int(gpu["count"]) == k
    if gpu.get("w") is not None:
        np.testing.assert_array_equal(np.asarray(gpu["w"])[:k], ref["w"][:k])
    if gpu.get("page_mask") is not None:
        m = np.asarray(gpu["page_mask"]).view(np.uint64)
        r = ref["page_mask"]
        n = min(m.size, r.size)
        np.testing.assert_array_equal(m[:n], r[:n])
        assert not m[n:].any()


def check_selection_tolerant(gpu_idx, gpu_count, or_scores, ref):
    """Index-set rule against the oracle's own scores."""
    k = int(ref["count"])
    assert int(gpu_count) == k, f"count {int(gpu_count)} != oracle {k}"
    g = set(int(j) for j in np.asarray(gpu_idx)[:k])
    o = set(int(j) for j in ref["idx"][:k])
    assert all(j >= 0 for j in g)
    if g == o:
        return 0
    s_kth = float(np.min(ref["w"][:k]))
    for j in g ^ o:
        assert abs(float(or_scores[j]) - s_kth) <= REL_TIE * abs(s_kth), \
            f"position {j} differs and is not a near-tie of the k-th score"
    return len(g ^ o)


def check_attention(gpu_out, or_out, gpu_lse=None, or_lse=None):
    """gpu_out bf16 tensor/array [..., D]; or_out fp64 oracle output."""
    g = np.asarray(torch.as_tensor(gpu_out).float().cpu(), np.float64)
    o = np.asarray(or_out, np.float64)
    err = np.abs(g - o)
    assert (err <= ATOL + RTOL * np.abs(o)).all(), f"max abs err {err.max():.3g}"
    if gpu_lse is not None:
        gl = np.asarray(torch.as_tensor(gpu_lse).float().cpu(), np.float64)
        fin = np.isfinite(or_lse)
        assert (np.isfinite(gl) == fin).all()
        assert np.abs(gl[fin] - or_lse[fin]).max(initial=0) < 1e-3
    return float(err.max()) if err.size else 0.0


def oracle_attend_rows(wc: W.Workload, idx_rows, scale=None):
    """Oracle attention of each row of a batch-1 workload over given idx rows."""
    sh = O.shape_of(wc, batch=1)
    return O.attend(sh, wc.q, wc.k_cache, wc.v_cache, wc.page_table,
                    np.asarray(idx_rows, np.int32).reshape(1, wc.num_q, -1), scale)
