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


# ------------------------------------------------------------ every row at once

def _hi(wc: W.Workload) -> int:
    return max(1, int(getattr(wc.config, "num_idx_heads", 1)))


def _positions(wc: W.Workload):
    """Query position of every selection row, [B, S_q * Hi] int64 (with
    several indexer heads, row r of a sequence is query row r // Hi)."""
    qs = wc.q_start.to(torch.int64).numpy()
    r = np.arange(wc.num_q * _hi(wc), dtype=np.int64)
    return qs[:, None] + (r // _hi(wc))[None, :]


def check_scores_all_rows(wc: W.Workload, g_scores, or_scores, exact=False, chunk_bytes=1 << 28):
    """Every causal score of every selection row within the fp32 bound
    (bit-exact with integer inputs), and nothing written past a row's query
    position. Scores are [B, S_q(, Hi), ld]. Returns the worst ratio of error
    to bound."""
    cfg = wc.config
    B = cfg.batch
    pos = _positions(wc)
    R = pos.shape[1]
    g_scores = np.asarray(g_scores).reshape(B, R, -1)
    or_scores = np.asarray(or_scores).reshape(B, R, -1)
    worst = 0.0
    for b in range(B):
        L = int(pos[b].max()) + 1
        K = np.abs(W.logical_rows(wc.k_comp_cache, wc.page_table, b, L).to(torch.float64).numpy())
        Q = np.abs(wc.q_comp[b].to(torch.float64).numpy()).reshape(R, cfg.d_c)
        step = max(1, chunk_bytes // (8 * L))
        for i0 in range(0, R, step):
            i1 = min(R, i0 + step)
            bound = gamma(cfg.d_c) * (Q[i0:i1] @ K.T)  # [rows, L]
            g = np.asarray(g_scores[b, i0:i1, :L], np.float64)
            o = np.asarray(or_scores[b, i0:i1, :L], np.float64)
            causal = np.arange(L)[None, :] <= pos[b, i0:i1, None]
            assert np.isnan(np.where(causal, 0.0, g)).sum() == (~causal).sum(), \
                f"sequence {b}: a score past the query position was written"
            if g_scores.shape[-1] > L:
                assert np.isnan(g_scores[b, i0:i1, L:]).all()
            if exact:
                assert np.array_equal(np.where(causal, g, 0.0), np.where(causal, o, 0.0)), \
                    f"sequence {b}: integer scores differ"
                continue
            err = np.where(causal, np.abs(g - o), 0.0)
            lim = np.where(causal, bound + U * np.abs(o), 1.0) + 1e-30
            ratio = float((err / lim).max(initial=0.0))
            assert (err <= lim).all(), f"sequence {b}: score error beyond the fp32 bound ({ratio:.3g})"
            worst = max(worst, ratio)
    return worst


def check_all_rows(wc: W.Workload, g_scores, g_sel, g_out, g_lse, topk=None, n_sel_pages=None,
                   scale=None, exact=False):
    """Every selection row (query row x indexer head) of a CPU workload
    against the oracle.

    g_scores: the GPU's scores [B, S_q(, Hi), ld] (numpy, NaN past each
              query), or None when the call under test computed them
              internally (the selection is then checked against the oracle's
              selection on the oracle's scores only);
    g_sel:    the GPU's selection, numpy arrays idx and w (and, if it has them,
              count and page_mask);
    g_out, g_lse: the GPU's attention over its own selection.
    Checks: scores within the fp32 bound; selection bit-exact against the
    oracle's selection on the GPU's own fp32 scores; index sets against the
    oracle's own scores by the near-tie rule (block pruning: identical page
    sets first); attention within 2e-2 + 1e-2|ref| of the oracle's attention
    over the GPU's index set. The attention error against the oracle's own
    index set is returned beside the others, not asserted (a near-tie swap
    changes the set the outputs are taken over)."""
    cfg = wc.config
    topk = cfg.topk if topk is None else topk
    nsp = cfg.n_sel_pages if n_sel_pages is None else n_sel_pages
    sh = O.shape_of(wc)
    B, S, Hi = cfg.batch, wc.num_q, _hi(wc)
    lead = (B, S) + ((Hi,) if Hi > 1 else ())
    R = S * Hi
    or_sc = O.index_scores(sh, wc.q_comp, wc.k_comp_cache, wc.page_table, wc.seq_lens, wc.q_start)
    rep = {"rows": B * R}
    g_idx = np.asarray(g_sel["idx"]).reshape(lead + (topk,))
    g_w = np.asarray(g_sel["w"]).reshape(lead + (topk,)) if g_sel.get("w") is not None else None
    if g_scores is not None:
        g_scores = np.asarray(g_scores).reshape(lead + (-1,))
        rep["score_worst_ratio"] = check_scores_all_rows(wc, g_scores, or_sc, exact)
        ref_g = O.topk_select(sh, g_scores, wc.seq_lens, wc.q_start, topk, nsp)
        np.testing.assert_array_equal(g_idx, ref_g["idx"])
        if g_w is not None:
            np.testing.assert_array_equal(g_w, ref_g["w"])
        if g_sel.get("count") is not None:
            np.testing.assert_array_equal(np.asarray(g_sel["count"]).reshape(lead), ref_g["count"])
        if g_sel.get("page_mask") is not None:
            np.testing.assert_array_equal(
                np.asarray(g_sel["page_mask"]).reshape(lead + (-1,)).view(np.uint64),
                ref_g["page_mask"])
    ref_o = O.topk_select(sh, or_sc, wc.seq_lens, wc.q_start, topk, nsp)
    flat = lambda a: None if a is None else np.asarray(a).reshape((B, R) + np.asarray(a).shape[len(lead):])
    gi, oi, osc = flat(g_idx), flat(ref_o["idx"]), flat(or_sc)
    ro = {k: flat(v) for k, v in ref_o.items() if v is not None}
    rg_pages = flat(ref_g["sel_pages"]) if (g_scores is not None and nsp > 0) else None
    differing = 0
    for b in range(B):
        for r in range(R):
            if np.array_equal(gi[b, r], oi[b, r]):
                continue
            if rg_pages is not None:
                assert set(rg_pages[b, r]) == set(ro["sel_pages"][b, r]), \
                    f"row ({b}, {r}): the kept pages differ"
            k = int(ro["count"][b, r])
            differing += check_selection_tolerant(gi[b, r], int((gi[b, r] >= 0).sum()), osc[b, r],
                                                  {k2: v[b, r] for k2, v in ro.items()})
            assert k == int((gi[b, r] >= 0).sum())
    rep["positions_differing_within_near_ties"] = differing
    out_g, lse_g = O.attend(sh, wc.q, wc.k_cache, wc.v_cache, wc.page_table, g_idx, scale)
    rep["attend_err_gpu_set"] = check_attention(g_out, out_g, g_lse, lse_g)
    out_o, _ = O.attend(sh, wc.q, wc.k_cache, wc.v_cache, wc.page_table, ref_o["idx"], scale)
    g = np.asarray(torch.as_tensor(g_out).float().cpu(), np.float64)
    e = np.abs(g - out_o)
    rep["attend_err_oracle_set"] = float(e.max()) if e.size else 0.0
    rep["attend_within_tol_oracle_set"] = bool((e <= ATOL + RTOL * np.abs(out_o)).all())
    return rep
