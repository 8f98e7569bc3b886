"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Small shapes span several tiles, every select path (all kept, LDS row, long
rows through the histogram + candidate path, block pruning) and ragged tails;
the five named workloads run at full size with every query row (every step of
the 1M-token stream) checked against the oracle.
"""
import dataclasses
import math
import os
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from top_index_selection_amd import _lib as T
from top_index_selection_amd import pipeline as PL
from top_index_selection_amd import workloads as W

from _checks import (check_all_rows, check_attention, check_scores, check_selection_exact,
                     check_selection_tolerant, compact, oracle_attend_rows, oracle_scores_row,
                     abs_dot_bound, select_on_scores)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T.lib()
    O.set_threads(min(16, os.cpu_count() or 1))
    yield


def gpu_workload(cfg, seed):
    return W.make_workload(cfg, seed, device=DEV)


def to_np(t):
    return t.detach().cpu().numpy()


def check_decode_workload(w, check_given_scores=True, attend=True):
    """Full decode pipeline on a workload, every sequence checked."""
    cfg = w.config
    B = cfg.batch
    say("scores", cfg.name, "B", B, "d_c", cfg.d_c, "topk", cfg.topk, "pruned", cfg.n_sel_pages)
    scores = PL.index_score(w)
    say("fused select")
    sel = PL.topk_select(w)
    say("select on given gpu scores")
    sel_given = PL.topk_select(w, scores=scores.contiguous())
    say("decode step")
    step = PL.decode_step(w)
    torch.cuda.synchronize()
    for key in ("idx", "w"):
        np.testing.assert_array_equal(to_np(sel[key]), to_np(sel_given[key]))
    np.testing.assert_array_equal(to_np(step["idx"]), to_np(sel["idx"]))
    np.testing.assert_array_equal(to_np(step["w"]), to_np(sel["w"]))
    out_sep, lse_sep = PL.gather_attend(w, sel["idx"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(step["out"].view(torch.int16)), to_np(out_sep.view(torch.int16)))
    exact = cfg.values == "int"
    sc_np = to_np(scores)
    for b in range(B):
        wc = compact(w, b)
        p = int(wc.q_start[0])
        or_sc = oracle_scores_row(wc)
        g_sc = sc_np[b, 0, : p + 1]
        check_scores(g_sc, or_sc, abs_dot_bound(wc), exact=exact)
        assert np.isnan(sc_np[b, 0, p + 1:]).all()
        ref_g = select_on_scores(g_sc, p, cfg.topk, cfg.n_sel_pages)
        check_selection_exact({"idx": to_np(sel["idx"][b, 0]), "w": to_np(sel["w"][b, 0]),
                               "count": to_np(sel["count"][b, 0]),
                               "page_mask": to_np(sel["page_mask"][b, 0])}, ref_g, cfg.topk)
        ref_o = select_on_scores(or_sc, p, cfg.topk, cfg.n_sel_pages)
        if cfg.n_sel_pages == 0:
            check_selection_tolerant(to_np(sel["idx"][b, 0]), to_np(sel["count"][b, 0]), or_sc,
                                     ref_o)
        if check_given_scores:
            # identical fp32 inputs on both sides: bit-exact selection
            given = torch.zeros_like(scores[b:b + 1])
            given[0, 0, : p + 1] = torch.from_numpy(or_sc).to(DEV)
            ws = compact(w, b, device=DEV)
            g2 = PL.topk_select(ws, scores=given)
            torch.cuda.synchronize()
            check_selection_exact({"idx": to_np(g2["idx"][0, 0]), "w": to_np(g2["w"][0, 0]),
                                   "count": to_np(g2["count"][0, 0]),
                                   "page_mask": to_np(g2["page_mask"][0, 0])}, ref_o, cfg.topk)
        if attend:
            out_or, lse_or = oracle_attend_rows(wc, to_np(sel["idx"][b, 0])[None])
            check_attention(step["out"][b, 0], out_or[0, 0], step["lse"][b, 0], lse_or[0, 0])
    return scores, sel, step


# ------------------------------------------------------------ small shapes

LENGTHS = (1, 63, 64, 65, 700, 4097, 12288, 12289, 20000, 33333)


@pytest.mark.parametrize("d_c,values,topk,heads", [
    (64, "normal", 256, 8), (128, "normal", 2048, 32), (128, "int", 2048, 20),
    (64, "int", 17, 64), (128, "normal", 1, 16), (64, "normal", 4096, 5),
    (128, "normal", 300, 1)])
def test_decode_paths_small(d_c, values, topk, heads):
    cfg = W.small_config(name=f"small_{d_c}_{values}_{topk}", batch=len(LENGTHS), lengths=LENGTHS,
                         d_c=d_c, num_heads=heads, topk=topk, values=values)
    check_decode_workload(gpu_workload(cfg, seed=topk + d_c))


SHORT_LENGTHS = (1, 63, 64, 65, 255, 256, 257, 700, 4095, 4096, 4097, 8191, 12287, 12288)


@pytest.mark.parametrize("topk", [1, 256, 2048, 4096])
def test_short_row_select_kernel_matches_general(topk):
    """When every row fits in LDS (page table at most 12288 positions wide) the
    selection runs in the short-row kernel; the same rows behind a wider page
    table (64 more columns, all unused) run in the general kernel. Both are
    checked against the oracle and must agree bit for bit."""
    cfg = W.small_config(name=f"short_rows_{topk}", batch=len(SHORT_LENGTHS),
                         lengths=SHORT_LENGTHS, d_c=128, num_heads=16, topk=topk)
    w = gpu_workload(cfg, seed=7 + topk)
    assert w.max_pages * 64 <= 12288
    check_decode_workload(w)
    pad = torch.full((w.page_table.shape[0], 64), -1, dtype=torch.int32, device=DEV)
    wide = W.Workload(**{**w.__dict__, "page_table": torch.cat([w.page_table, pad], 1).contiguous(),
                         "max_pages": w.max_pages + 64})
    a = PL.decode_step(w)
    b = PL.decode_step(wide)
    torch.cuda.synchronize()
    bits = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.int32: torch.int32}
    for k in ("idx", "w", "out", "lse"):
        assert torch.equal(a[k].view(bits[a[k].dtype]), b[k].view(bits[b[k].dtype])), k


def test_small_launch_scorer_blocks_are_invisible():
    """14 short rows make a launch smaller than one 16-page block per compute
    unit, so they are scored one page per wave; the same rows followed by 10
    more make it large enough for 16-page blocks. The first 14 rows' results
    must be the same bit for bit."""
    lengths = SHORT_LENGTHS + (12288,) * 10
    cfg = W.small_config(name="small_launch", batch=len(lengths), lengths=lengths, d_c=64,
                         num_heads=8, topk=256)
    w = gpu_workload(cfg, seed=5)
    assert w.max_pages == 192 and len(lengths) * 12 >= 256 > len(SHORT_LENGTHS) * 12
    nb = len(SHORT_LENGTHS)
    head = W.Workload(**{**w.__dict__, "config": dataclasses.replace(cfg, batch=nb),
                         "seq_lens": w.seq_lens[:nb].contiguous(), "q_start": w.q_start[:nb].contiguous(),
                         "page_table": w.page_table[:nb].contiguous(), "q_comp": w.q_comp[:nb].contiguous(),
                         "q": w.q[:nb].contiguous()})
    check_decode_workload(head)
    a = PL.decode_step(head)
    b = PL.decode_step(w)
    torch.cuda.synchronize()
    bits = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.int32: torch.int32}
    for k in ("idx", "w", "out", "lse"):
        assert torch.equal(a[k].view(bits[a[k].dtype]), b[k][:nb].view(bits[b[k].dtype])), k


def test_scorer_block_width_is_invisible():
    """Long rows behind a page table of their own width are scored in 32-page
    blocks (one round of blocks covers the table); behind a table widened to
    10,000 pages, in 24-page blocks. Scores, selections and outputs must be
    the same bit for bit, and match the oracle."""
    cfg = W.small_config(name="block_width", batch=3, lengths=(20000, 40000, 70001), d_c=128,
                         num_heads=32, topk=2048)
    w = gpu_workload(cfg, seed=11)
    check_decode_workload(w)
    pad = torch.full((w.page_table.shape[0], 10000 - w.max_pages), -1, dtype=torch.int32,
                     device=DEV)
    wide = W.Workload(**{**w.__dict__, "page_table": torch.cat([w.page_table, pad], 1).contiguous(),
                         "max_pages": 10000})
    a = PL.decode_step(w)
    b = PL.decode_step(wide)
    torch.cuda.synchronize()
    bits = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.int32: torch.int32}
    for k in ("idx", "w", "out", "lse"):
        assert torch.equal(a[k].view(bits[a[k].dtype]), b[k].view(bits[b[k].dtype])), k


@pytest.mark.parametrize("n_sel,topk,values", [(1, 64, "normal"), (5, 300, "normal"),
                                               (64, 2048, "normal"), (7, 200, "int"),
                                               (192, 4096, "normal")])
def test_block_pruned_small(n_sel, topk, values):
    cfg = W.small_config(name="pruned", batch=5, lengths=(100, 1000, 5000, 40000, 70001), d_c=128,
                         num_heads=32, topk=topk, n_sel_pages=n_sel, values=values,
                         shift_frac=0.25, shift_value=0.5)
    check_decode_workload(gpu_workload(cfg, seed=n_sel))


@pytest.mark.parametrize("d_c", [128, 64])
def test_block_pruned_one_round_scorer(d_c):
    """Block pruning over a table wide enough for the page-maxima scorer that
    holds a block's scores in LDS until the block ends (one round of blocks of
    about 24 pages here): ragged rows, partial last pages, rows of one page
    and of one token."""
    lengths = (131072, 100000, 70001, 4097, 65, 1, 120000, 98303)
    cfg = W.small_config(name="pruned_wide", batch=len(lengths), lengths=lengths, d_c=d_c,
                         num_heads=32, topk=2048, n_sel_pages=64, values="normal",
                         shift_frac=0.25, shift_value=0.5)
    check_decode_workload(gpu_workload(cfg, seed=d_c))


@pytest.mark.parametrize("case", ["prefill", "prefill_long_rows", "decode", "pruned",
                                  "pruned_one_round", "multihead"])
def test_select_outputs_do_not_depend_on_the_page_mask(case):
    """Without a page mask to build, the selection writes its kept entries
    straight to idx and w; with one they pass through LDS. Both give the same
    idx, w and count bit for bit on every path: short prefill rows, prefill
    rows longer than the LDS key buffer, short, candidate (up to and over 32
    slices) and all-kept decode rows, block pruning on small and one-round
    tables, several indexer heads; and idx alone when w is not asked for."""
    cfgs = {
        "prefill": W.small_config(name="pm_pf", batch=2, lengths=(3000, 3000), prefill=True,
                                  d_c=64, topk=256),
        "prefill_long_rows": W.small_config(name="pm_pfl", batch=1, lengths=(9000,), prefill=True,
                                            d_c=64, topk=2048),
        "decode": W.small_config(name="pm_dec", batch=6,
                                 lengths=(1000, 5000, 13000, 40000, 131072, 200000), d_c=128,
                                 num_heads=32, topk=2048),
        "pruned": W.small_config(name="pm_pr", batch=3, lengths=(100, 70001, 262144), d_c=128,
                                 num_heads=32, topk=2048, n_sel_pages=64, shift_frac=0.25,
                                 shift_value=0.5),
        "pruned_one_round": W.small_config(name="pm_pr1", batch=8, lengths=(131072,) * 7 + (98303,),
                                           d_c=128, num_heads=32, topk=2048, n_sel_pages=64),
        "multihead": W.small_config(name="pm_mh", batch=3, lengths=(700, 20000, 90000), d_c=128,
                                    num_heads=32, topk=1024, num_idx_heads=4),
    }
    w = gpu_workload(cfgs[case], seed=3)
    say(f"page-mask independence: {case}")
    with_mask = PL.topk_select(w)
    without = PL.topk_select(w, page_mask=False)
    idx_only = PL.topk_select(w, page_mask=False, weights=False)
    mask_only = PL.topk_select(w, weights=False)
    torch.cuda.synchronize()
    assert torch.equal(with_mask["idx"], without["idx"])
    assert torch.equal(with_mask["w"].view(torch.int32), without["w"].view(torch.int32))
    assert torch.equal(with_mask["count"], without["count"])
    # without w the prefill scorer leaves out the rows that keep every position
    for other in (idx_only, mask_only):
        assert torch.equal(with_mask["idx"], other["idx"])
        assert torch.equal(with_mask["count"], other["count"])
    assert torch.equal(with_mask["page_mask"], mask_only["page_mask"])


def test_empty_sequences_in_a_batch():
    """Sequences that hold no tokens yet (seq_lens 0) have no query position and
    no candidates: their rows select nothing (count 0, idx all -1, w 0) and
    attend to nothing (out 0, lse -inf), as the oracle gives for an empty
    candidate set, while the other rows of the batch (ragged, long and short)
    keep their results."""
    lengths = (0, 1, 20000, 0, 700)
    cfg = W.small_config(name="empty", batch=len(lengths), lengths=lengths, d_c=128,
                         num_heads=32, topk=256)
    w = gpu_workload(cfg, seed=5)
    say("empty sequences: scores, select, decode step")
    scores = PL.index_score(w)
    sel = PL.topk_select(w)
    step = PL.decode_step(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(step["idx"]), to_np(sel["idx"]))
    sc_np = to_np(scores)
    for b, L in enumerate(lengths):
        if L == 0:
            assert np.isnan(sc_np[b, 0]).all()  # nothing scored
            assert int(sel["count"][b, 0]) == 0
            assert (to_np(sel["idx"][b, 0]) == -1).all()
            assert (to_np(sel["w"][b, 0]) == 0).all()
            assert (to_np(sel["page_mask"][b, 0]) == 0).all()
            assert (to_np(step["out"][b, 0].float()) == 0).all()
            assert np.isneginf(to_np(step["lse"][b, 0])).all()
            continue
        wc = compact(w, b)
        p = int(wc.q_start[0])
        g_sc = sc_np[b, 0, : p + 1]
        check_scores(g_sc, oracle_scores_row(wc), abs_dot_bound(wc))
        ref_g = select_on_scores(g_sc, p, cfg.topk, 0)
        check_selection_exact({"idx": to_np(sel["idx"][b, 0]), "w": to_np(sel["w"][b, 0]),
                               "count": to_np(sel["count"][b, 0]),
                               "page_mask": to_np(sel["page_mask"][b, 0])}, ref_g, cfg.topk)
        out_or, lse_or = oracle_attend_rows(wc, to_np(sel["idx"][b, 0])[None])
        check_attention(step["out"][b, 0], out_or[0, 0], step["lse"][b, 0], lse_or[0, 0])
    # the oracle's own reading of an empty row
    wc = compact(w, 0)
    out_or, lse_or = oracle_attend_rows(wc, np.full((1, cfg.topk), -1, np.int32))
    assert (out_or == 0).all() and np.isneginf(lse_or).all()


def test_page_granular_attention():
    """Whole-page attention: with topk = n_sel_pages * block_size the pruned
    selection keeps every token of the best pages, and the attention runs over
    those pages in full. The kept set must be exactly the union of the pages
    the oracle ranks first by page maximum (ties: lower page)."""
    n_sel = 24
    cfg = W.small_config(name="page_attn", batch=3, lengths=(5000, 40000, 70001), d_c=128,
                         num_heads=32, topk=n_sel * 64, n_sel_pages=n_sel, shift_frac=0.25,
                         shift_value=0.5)
    w = gpu_workload(cfg, seed=21)
    scores = PL.index_score(w)
    step = PL.decode_step(w)
    torch.cuda.synchronize()
    for b in range(cfg.batch):
        wc = compact(w, b)
        p = int(wc.q_start[0])
        g_sc = to_np(scores[b, 0, : p + 1])
        ref = select_on_scores(g_sc, p, cfg.topk, n_sel)
        pages = sorted(ref["sel_pages"])
        want = [j for g in pages for j in range(g * 64, min(g * 64 + 64, p + 1))]
        got = to_np(step["idx"][b, 0])
        np.testing.assert_array_equal(got[: len(want)], np.array(want, np.int32))
        assert (got[len(want):] == -1).all()
        out_or, lse_or = oracle_attend_rows(wc, got[None])
        check_attention(step["out"][b, 0], out_or[0, 0], step["lse"][b, 0], lse_or[0, 0])


def test_block_pruned_keeps_exact_topk_when_pages_cover_it():
    cfg = W.small_config(name="pruned_exact", batch=2, lengths=(3000, 9000), d_c=64,
                         num_heads=8, topk=64, n_sel_pages=64)
    w = gpu_workload(cfg, 5)
    a = PL.topk_select(w)
    b = PL.topk_select(w, n_sel_pages=0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(a["idx"]), to_np(b["idx"]))


@pytest.mark.parametrize("L,d_c,topk,values,heads", [
    (700, 64, 256, "normal", 16), (2100, 128, 2048, "normal", 32), (1000, 64, 100, "int", 48),
    (300, 128, 4096, "normal", 8), (900, 64, 200, "normal", 1)])
def test_prefill_small(L, d_c, topk, values, heads):
    cfg = W.small_config(name="prefill", batch=1, lengths=(L,), prefill=True, d_c=d_c,
                         num_heads=heads, topk=topk, values=values)
    w = gpu_workload(cfg, seed=L)
    say("prefill scores", L, d_c, topk, values)
    scores = PL.index_score(w)
    sel = PL.topk_select(w)
    sel_given = PL.topk_select(w, scores=scores)
    out, lse = PL.gather_attend(w, sel["idx"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(sel["idx"]), to_np(sel_given["idx"]))
    wc = W.to_device(w, "cpu")
    rep = check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()}, out, to_np(lse),
                         exact=values == "int")
    _report(f"prefill L={L}", rep)


def test_prefill_attention_without_lse_output():
    """Without an lse output the prefill attention keeps no fp32 weight sum;
    the attention output itself does not depend on it and stays bitwise equal
    (16 and 40 heads: one and three head tiles)."""
    for heads in (16, 40):
        cfg = W.small_config(name="nolse", batch=1, lengths=(2600,), prefill=True, d_c=64,
                             num_heads=heads, topk=1024)
        w = gpu_workload(cfg, seed=heads)
        sel = PL.topk_select(w)
        out_lse, lse = PL.gather_attend(w, sel["idx"])
        out = torch.empty_like(out_lse)
        T.paged_gather_attend(PL.shape_of(w), T.TIS_PHASE_PREFILL, w.q, w.k_cache, w.v_cache,
                              w.page_table, sel["idx"], cfg.topk, 0.0, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(out.view(torch.int16)), to_np(out_lse.view(torch.int16)))
        assert np.isfinite(to_np(lse)).all()


@pytest.mark.parametrize("phase,scale", [(T.TIS_PHASE_DECODE, 0.05), (T.TIS_PHASE_PREFILL, 0.05),
                                         (T.TIS_PHASE_DECODE, 0.3), (T.TIS_PHASE_PREFILL, 0.3)])
def test_caller_softmax_scale(phase, scale):
    """A softmax scale passed by the caller replaces 1/sqrt(head_dim) in the
    logits and in lse, on both attention paths."""
    prefill = phase == T.TIS_PHASE_PREFILL
    lengths = (1500,) if prefill else (3000, 20000, 777)
    cfg = W.small_config(name="scale", batch=len(lengths), lengths=lengths, prefill=prefill,
                         d_c=64, num_heads=24, topk=512)
    w = gpu_workload(cfg, seed=int(scale * 100) + phase)
    sel = PL.topk_select(w)
    out, lse = PL.gather_attend(w, sel["idx"], phase=phase, scale=scale)
    out_d, lse_d = PL.gather_attend(w, sel["idx"], phase=phase)
    torch.cuda.synchronize()
    wc = W.to_device(w, "cpu")
    sh = O.shape_of(wc)
    idx = to_np(sel["idx"])
    out_or, lse_or = O.attend(sh, wc.q, wc.k_cache, wc.v_cache, wc.page_table, idx, scale)
    err = check_attention(out, out_or, to_np(lse), lse_or)
    out_or_d, lse_or_d = O.attend(sh, wc.q, wc.k_cache, wc.v_cache, wc.page_table, idx)
    check_attention(out_d, out_or_d, to_np(lse_d), lse_or_d)
    # the override is not silently ignored: lse differs from the default's
    fin = np.isfinite(lse_or)
    assert np.abs(lse_or[fin] - lse_or_d[fin]).max() > 1e-2
    say("caller scale", scale, "phase", phase, "max out err", err)


def test_prefill_batched_64_heads():
    """Three sequences, 64 heads: the mask-scheduled prefill kernel then holds 4
    rows of 4 head tiles per workgroup and takes the sequence from the block."""
    cfg = W.small_config(name="prefill_b3", batch=3, lengths=(1500, 1500, 1500), prefill=True,
                         d_c=128, num_heads=64, topk=300)
    w = gpu_workload(cfg, seed=11)
    say("prefill batch 3, 64 heads")
    scores = PL.index_score(w)
    sel = PL.topk_select(w)
    out, lse = PL.gather_attend(w, sel["idx"])
    torch.cuda.synchronize()
    wc = W.to_device(w, "cpu")
    _report("prefill batch 3", check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()},
                                              out, to_np(lse)))


def test_prefill_chunk_with_q_start():
    """Chunked prefill: 500 query rows at positions 2500..2999 of a 3000-token
    cache (q_start = 2500), through scoring, selection and attention."""
    base = gpu_workload(W.small_config(name="prefill_chunk", batch=1, lengths=(3000,), prefill=True,
                                       d_c=64, num_heads=16, topk=700), seed=12)
    w = W.Workload(**{**base.__dict__, "num_q": 500,
                      "q_start": torch.tensor([2500], dtype=torch.int32, device=DEV),
                      "q_comp": base.q_comp[:, 2500:].contiguous(), "q": base.q[:, 2500:].contiguous()})
    say("prefill chunk at 2500")
    scores = PL.index_score(w)
    sel = PL.topk_select(w)
    sel_given = PL.topk_select(w, scores=scores)
    out, lse = PL.gather_attend(w, sel["idx"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(sel["idx"]), to_np(sel_given["idx"]))
    wc = W.to_device(w, "cpu")
    _report("prefill chunk", check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()},
                                            out, to_np(lse)))


@pytest.mark.parametrize("hi", [1, 4])
def test_prefill_index_only_selection_on_a_ragged_batch(hi):
    """2500 prefill rows per sequence, each sequence's rows ending at its last
    token (q_start = seq_len - 2500): an empty sequence (every row before
    position 0: no candidates), a 1000-token one (its first 1500 rows have
    none) and a 2500-token one, with one or four indexer heads (the last
    64-row block is ragged). Asked for the index lists alone, the scorer
    leaves out the row blocks whose rows all see at most topk positions and
    the selection keeps all of such a row unread; the lists and counts equal
    those of the call that also returns w (every row scored), which are
    checked against the oracle."""
    base = gpu_workload(W.small_config(name=f"pf_ragged{hi}", batch=3, lengths=(2500,) * 3,
                                       prefill=True, d_c=64, num_heads=32, topk=300,
                                       num_idx_heads=hi), seed=21 + hi)
    lens = torch.tensor([0, 1000, 2500], dtype=torch.int32, device=DEV)
    w = W.Workload(**{**base.__dict__, "seq_lens": lens, "q_start": lens - base.num_q})
    say("prefill index-only selection, ragged batch, indexer heads", hi)
    full = PL.topk_select(w)
    idx_only = PL.topk_select(w, page_mask=False, weights=False)
    out, lse = PL.gather_attend(w, full["idx"])
    torch.cuda.synchronize()
    assert torch.equal(full["idx"], idx_only["idx"])
    assert torch.equal(full["count"], idx_only["count"])
    assert int(full["count"][0].max()) == 0  # the empty sequence selects nothing
    wc = W.to_device(w, "cpu")
    _report(f"prefill ragged batch hi={hi}",
            check_all_rows(wc, None, {k: to_np(v) for k, v in full.items()}, out, to_np(lse)))


def test_prefill_long_context_fallbacks():
    """Prefill over 258 pages at topk 64: the attention takes the per-row
    gather (a sparse selection), and rows longer than 8192 positions are
    selected from the global score row (first-digit histogram, then the
    candidates in LDS)."""
    L = 16500
    cfg = W.small_config(name="prefill_long", batch=1, lengths=(L,), prefill=True, d_c=64,
                         num_heads=16, topk=64)
    w = gpu_workload(cfg, seed=7)
    assert w.max_pages > 256
    say("prefill long", L)
    scores = PL.index_score(w)
    sel = PL.topk_select(w, scores=scores)
    out, lse = PL.gather_attend(w, sel["idx"])
    torch.cuda.synchronize()
    wc = W.to_device(w, "cpu")
    _report("prefill long", check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()},
                                           out, to_np(lse)))
    say("prefill long ok")


@pytest.mark.parametrize("L,rows,topk", [(40000, 300, 2048), (20000, 200, 4096), (12000, 2048, 4096)])
def test_prefill_chunk_of_a_long_context(L, rows, topk):
    """The last query rows of a long cache: rows longer than the select's LDS
    key buffer are selected from a first-digit histogram of the score row and
    the candidates gathered into LDS; the attention takes the per-row gather
    where the rows' contexts average more than 4 x topk positions (40000 and
    20000 tokens) and otherwise the mask-scheduled kernel, here walking the
    context in two windows of pages (12000 tokens, 188 pages, 2048 rows at
    topk 4096)."""
    base = gpu_workload(W.small_config(name="prefill_long_chunk", batch=1, lengths=(L,),
                                       prefill=True, d_c=64, num_heads=32, topk=topk), seed=17)
    w = W.Workload(**{**base.__dict__, "num_q": rows,
                      "q_start": torch.tensor([L - rows], dtype=torch.int32, device=DEV),
                      "q_comp": base.q_comp[:, L - rows:].contiguous(),
                      "q": base.q[:, L - rows:].contiguous()})
    assert w.max_pages > 128
    say("prefill chunk at", L - rows, "of", L, "topk", topk)
    scores = PL.index_score(w)
    sel = PL.topk_select(w, scores=scores)
    sel_fused = PL.topk_select(w)
    out, lse = PL.gather_attend(w, sel["idx"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(sel["idx"]), to_np(sel_fused["idx"]))
    wc = W.to_device(w, "cpu")
    _report("prefill long chunk", check_all_rows(wc, to_np(scores),
                                                 {k: to_np(v) for k, v in sel.items()}, out,
                                                 to_np(lse)))


def test_attention_closed_forms():
    cfg = W.small_config(name="closed", batch=3, lengths=(50, 300, 5000), d_c=64, num_heads=24,
                         topk=128)
    w = gpu_workload(cfg, 3)
    sel = PL.topk_select(w)
    idx = sel["idx"]
    # one selected position: the output is that V row exactly
    one = torch.full_like(idx, -1)
    one[..., 0] = idx[..., 5]
    out, lse = PL.gather_attend(w, one)
    torch.cuda.synchronize()
    for b in range(3):
        j = int(idx[b, 0, 5])
        vrow = W.logical_rows(w.v_cache, w.page_table, b, j + 1)[j]
        for h in range(24):
            assert torch.equal(out[b, 0, h], vrow)
    # constant V: exactly that constant
    wv = W.Workload(**{**w.__dict__, "v_cache": torch.full_like(w.v_cache, -1.625)})
    out, _ = PL.gather_attend(wv, idx)
    torch.cuda.synchronize()
    assert (out.float() == -1.625).all()
    # q = 0: the mean of the selected V rows
    wq = W.Workload(**{**w.__dict__, "q": torch.zeros_like(w.q)})
    out, lse = PL.gather_attend(wq, idx)
    torch.cuda.synchronize()
    for b in range(3):
        k = int(sel["count"][b, 0])
        rows = W.logical_rows(w.v_cache, w.page_table, b, int(w.seq_lens[b]))
        mean = rows[idx[b, 0, :k].long()].double().mean(0)
        assert (out[b, 0].double() - mean).abs().max() < 1e-2
        assert torch.allclose(lse[b, 0].double(), torch.full_like(lse[b, 0].double(), math.log(k)),
                              atol=1e-4)
    # no selected position: zeros and lse = -inf
    none = torch.full_like(idx, -1)
    out, lse = PL.gather_attend(w, none)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()
    # topk >= context: equals the oracle's dense causal attention
    wc = compact(w, 0)
    sh = O.shape_of(wc)
    dense, _ = O.dense_causal_attention(sh, wc.q, wc.k_cache, wc.v_cache, wc.page_table,
                                        wc.seq_lens, wc.q_start)
    check_attention(out_dense := PL.decode_step(w)["out"][0, 0], dense[0, 0])


def test_split_count_does_not_change_results_beyond_rounding():
    cfg = W.small_config(name="splits", batch=1, lengths=(9000,), d_c=128, num_heads=64,
                         topk=2048)
    w = gpu_workload(cfg, 1)
    sel = PL.topk_select(w)
    dec, _ = PL.gather_attend(w, sel["idx"], phase=T.TIS_PHASE_DECODE)
    pre, _ = PL.gather_attend(w, sel["idx"], phase=T.TIS_PHASE_PREFILL)
    torch.cuda.synchronize()
    assert (dec.float() - pre.float()).abs().max() < 2e-2


# ----------------------------------------------------------- structure

def test_page_permutation_is_bitwise_invisible():
    cfg = W.small_config(name="perm", batch=3, lengths=(5000, 20000, 130), d_c=128,
                         num_heads=32, topk=512)
    w = gpu_workload(cfg, 2)
    w2 = W.permute_pool(w, 77)
    a, b = PL.decode_step(w), PL.decode_step(w2)
    torch.cuda.synchronize()
    for k in ("idx", "w", "lse"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))


def test_run_twice_bitwise():
    cfg = W.small_config(name="twice", batch=4, lengths=(40000, 100, 13000, 5000), d_c=128,
                         num_heads=32, topk=2048)
    w = gpu_workload(cfg, 9)
    ws = torch.empty(T.workspace_size(PL.shape_of(w), T.TIS_OP_DECODE_STEP, 2048, 0),
                     dtype=torch.uint8, device=DEV)
    a = {k: v.clone() for k, v in PL.decode_step(w, workspace=ws).items()}
    b = PL.decode_step(w, workspace=ws)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k]), k


def test_planted_key_is_selected():
    cfg = W.small_config(name="planted", batch=2, lengths=(30000, 3000), d_c=128, num_heads=16,
                         topk=64)
    w = gpu_workload(cfg, 4)
    for b, j in ((0, 12345), (1, 7)):
        row = W.logical_rows(w.k_comp_cache, w.page_table, b, j + 1)
        page = int(w.page_table[b, j // 64])
        w.k_comp_cache[page, j % 64] = (8.0 * w.q_comp[b, 0].float()).to(torch.bfloat16)
    sel = PL.topk_select(w)
    torch.cuda.synchronize()
    assert 12345 in to_np(sel["idx"][0, 0]) and 7 in to_np(sel["idx"][1, 0])


def test_all_scores_tied_on_long_rows():
    """q_comp = 0 makes every score zero (+0 or -0, which compare equal): the
    tie rule then keeps exactly the K' lowest positions. On rows longer than the
    LDS capacity the threshold bin holds every position, more candidates than
    the candidate path takes, so the selection runs over the score row in
    global memory; the oracle gives the same sets."""
    lengths = (20000, 13000, 40000, 5000)
    cfg = W.small_config(name="tied", batch=len(lengths), lengths=lengths, d_c=128,
                         num_heads=16, topk=2048)
    w = gpu_workload(cfg, seed=9)
    w.q_comp.zero_()
    scores = PL.index_score(w)
    sel = PL.topk_select(w)
    step = PL.decode_step(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(step["idx"]), to_np(sel["idx"]))
    sc_np = to_np(scores)
    for b, L in enumerate(lengths):
        k = min(L, cfg.topk)
        assert (sc_np[b, 0, :L] == 0).all()
        np.testing.assert_array_equal(to_np(sel["idx"][b, 0, :k]), np.arange(k))
        assert int(sel["count"][b, 0]) == k
        assert (to_np(sel["w"][b, 0]) == 0).all()
        ref = select_on_scores(sc_np[b, 0, :L], L - 1, cfg.topk, 0)
        check_selection_exact({"idx": to_np(sel["idx"][b, 0]), "w": to_np(sel["w"][b, 0]),
                               "count": to_np(sel["count"][b, 0]),
                               "page_mask": to_np(sel["page_mask"][b, 0])}, ref, cfg.topk)
        wc = compact(w, b)
        out_or, lse_or = oracle_attend_rows(wc, to_np(sel["idx"][b, 0])[None])
        check_attention(step["out"][b, 0], out_or[0, 0], step["lse"][b, 0], lse_or[0, 0])


# ----------------------------------------------------- named workloads

def test_config_decode_4k():
    w = gpu_workload(W.CONFIGS["decode_4k"], 0)
    check_decode_workload(w)


def _report(name, rep):
    say(name, "every row checked:", {k: (round(v, 4) if isinstance(v, float) else v)
                                     for k, v in rep.items()})


def _full_decode_check(w):
    """Scores, fused selection and decode step of a full-size decode workload,
    every sequence checked against the oracle."""
    cfg = w.config
    scores = PL.index_score(w)
    sel = PL.topk_select(w)
    step = PL.decode_step(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(step["idx"]), to_np(sel["idx"]))
    np.testing.assert_array_equal(to_np(step["w"]), to_np(sel["w"]))
    wc = W.to_device(w, "cpu")
    rep = check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()},
                         step["out"], to_np(step["lse"]))
    _report(cfg.name, rep)
    return rep


@pytest.mark.parametrize("seed", [0, 1])
def test_config_batched_decode_32k_128k(seed):
    w = gpu_workload(W.CONFIGS["batched_decode_32k_128k"], seed)
    say("batched decode full size, seed", seed)
    _full_decode_check(w)


def test_config_block_pruned_256k():
    w = gpu_workload(W.CONFIGS["block_pruned_256k"], 0)
    say("block pruned full size")
    _full_decode_check(w)


def test_config_prefill_8k():
    w = gpu_workload(W.CONFIGS["prefill_8k"], 0)
    cfg = w.config
    say("prefill full size")
    scores = PL.index_score(w)
    sel = PL.topk_select(w, scores=scores)
    out, lse = PL.gather_attend(w, sel["idx"])
    sel_fused = PL.topk_select(w)
    # the launch the benchmark times: index lists only (no w, no page mask)
    sel_bench = PL.topk_select(w, page_mask=False, weights=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(sel["idx"]), to_np(sel_fused["idx"]))
    np.testing.assert_array_equal(to_np(sel["idx"]), to_np(sel_bench["idx"]))
    wc = W.to_device(w, "cpu")
    rep = check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()}, out, to_np(lse))
    _report(cfg.name, rep)
    # rows 0..topk-1 keep every valid position: dense causal attention
    n = cfg.topk
    sh = O.shape_of(wc, num_q=n)
    dense, dense_lse = O.dense_causal_attention(sh, wc.q[:, :n], wc.k_cache, wc.v_cache,
                                                wc.page_table, None, wc.q_start)
    check_attention(out[:, :n], dense, lse[:, :n], dense_lse)
    say("rows 0 ..", n - 1, "equal dense causal attention")


def test_config_long_decode_1m_stream():
    w = gpu_workload(W.CONFIGS["long_decode_1m"], 0)
    cfg = w.config
    T_steps = cfg.stream_steps
    L0 = int(w.seq_lens[0])
    cap = w.max_pages * cfg.block_size
    say("1M stream: pre-filled", L0, "steps", T_steps)
    # one-shot cache: every appended row written straight into its slot
    one_shot = {k: getattr(w, k).clone() for k in ("k_comp_cache", "k_cache", "v_cache")}
    for t in range(T_steps):
        pos = L0 + t
        page = int(w.page_table[0, pos // 64])
        one_shot["k_comp_cache"][page, pos % 64] = w.stream.k_comp_new[t, 0]
        one_shot["k_cache"][page, pos % 64] = w.stream.k_new[t, 0]
        one_shot["v_cache"][page, pos % 64] = w.stream.v_new[t, 0]
    ws = torch.empty(T.workspace_size(PL.shape_of(w), T.TIS_OP_DECODE_STEP, cfg.topk, 0),
                     dtype=torch.uint8, device=DEV)
    g_sc = torch.empty((T_steps, cap), dtype=torch.float32, device=DEV)
    keep = {k: [] for k in ("idx", "w", "out", "lse")}
    for t in range(T_steps):
        PL.append(w, t)
        wt = W.Workload(**{**w.__dict__, "q_comp": w.stream.q_comp[t], "q": w.stream.q[t]})
        res = PL.decode_step(wt, workspace=ws)
        for k in keep:
            keep[k].append(res[k][0, 0].clone())
        g_sc[t] = PL.index_score(wt, q_start=None)[0, 0]
    torch.cuda.synchronize()
    assert int(w.seq_lens[0]) == L0 + T_steps
    for k in one_shot:
        assert torch.equal(getattr(w, k).view(torch.int16), one_shot[k].view(torch.int16)), k
    say("stream done; checking all", T_steps, "steps")
    # Every step as one row of a single problem over the final cache: step t's
    # query sits at L0 + t and sees positions 0..L0+t only, all of which were
    # in the cache when the step ran.
    wc = compact(w, 0)
    wc = W.Workload(**{**wc.__dict__, "num_q": T_steps,
                       "q_comp": w.stream.q_comp[:, 0, 0].unsqueeze(0).cpu(),
                       "q": w.stream.q[:, 0, 0].unsqueeze(0).cpu(),
                       "q_start": torch.tensor([L0], dtype=torch.int32),
                       "seq_lens": torch.tensor([L0 + T_steps], dtype=torch.int32)})
    g_sel = {"idx": torch.stack(keep["idx"]).cpu().numpy()[None],
             "w": torch.stack(keep["w"]).cpu().numpy()[None]}
    rep = check_all_rows(wc, g_sc.cpu().numpy()[None], g_sel, torch.stack(keep["out"])[None],
                         torch.stack(keep["lse"]).cpu().numpy()[None])
    _report(cfg.name, rep)
