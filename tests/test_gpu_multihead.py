"""Several indexer heads on the GPU against the oracle (needs an MI355X).

Each (query row, indexer head) selects its own top-k over the shared
compressed keys, and query head h attends over the set of indexer head
h // (H / Hi) ("Day-0 Inference Adaptation of Ultra-Large-Scale MoE Models on
Domestic AI Accelerators", section 4.1: scores [B, H, S, S_c], top-k along
the last axis). Every selection row of every case is checked.
"""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from top_index_selection_amd import _lib as T
from top_index_selection_amd import pipeline as PL
from top_index_selection_amd import workloads as W

from _checks import check_all_rows

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


def to_np(t):
    return t.detach().cpu().numpy()


def _decode_case(cfg, seed):
    w = W.make_workload(cfg, seed, device=DEV)
    scores = PL.index_score(w)
    sel = PL.topk_select(w)
    sel_given = PL.topk_select(w, scores=scores.contiguous())
    step = PL.decode_step(w)
    out_sep, lse_sep = PL.gather_attend(w, sel["idx"])
    torch.cuda.synchronize()
    for k in ("idx", "w", "count", "page_mask"):
        np.testing.assert_array_equal(to_np(sel[k]), to_np(sel_given[k]))
    np.testing.assert_array_equal(to_np(step["idx"]), to_np(sel["idx"]))
    np.testing.assert_array_equal(to_np(step["w"]), to_np(sel["w"]))
    np.testing.assert_array_equal(to_np(step["out"].view(torch.int16)),
                                  to_np(out_sep.view(torch.int16)))
    wc = W.to_device(w, "cpu")
    rep = check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()}, step["out"],
                         to_np(step["lse"]), exact=cfg.values == "int")
    say(cfg.name, rep)
    return w, sel


LENGTHS = (1, 63, 700, 4097, 12288, 12289, 33333)


@pytest.mark.parametrize("hi,heads,d_c,topk,values", [
    (2, 32, 128, 2048, "normal"), (4, 64, 128, 256, "normal"), (16, 16, 64, 512, "normal"),
    (3, 24, 64, 100, "int"), (8, 64, 128, 4096, "normal")])
def test_multihead_decode_small(hi, heads, d_c, topk, values):
    cfg = W.small_config(name=f"mh{hi}_{d_c}_{topk}", batch=len(LENGTHS), lengths=LENGTHS,
                         d_c=d_c, num_heads=heads, topk=topk, values=values, num_idx_heads=hi,
                         kcomp_scale=1.0 if values == "int" else 1.0 / np.sqrt(d_c))
    w, sel = _decode_case(cfg, seed=hi * 10 + d_c)
    # the heads choose different sets (else a head mix-up could pass unseen)
    idx = to_np(sel["idx"])
    assert not np.array_equal(idx[-1, 0, 0], idx[-1, 0, 1])


def test_multihead_block_pruned():
    cfg = W.small_config(name="mh_pruned", batch=3, lengths=(9000, 64, 30000), d_c=128,
                         num_heads=32, topk=512, n_sel_pages=12, num_idx_heads=4,
                         shift_frac=0.25, shift_value=0.5)
    _decode_case(cfg, seed=5)


def test_zero_indexer_heads_read_as_one():
    cfg = W.small_config(name="mh_zero", batch=2, lengths=(5000, 20000), d_c=128, num_heads=16,
                         topk=1024)
    w = W.make_workload(cfg, 3, device=DEV)
    ref = PL.decode_step(w)
    sh = PL.shape_of(w)
    sh.num_idx_heads = 0
    out = torch.empty_like(ref["out"])
    idx = torch.empty_like(ref["idx"])
    T.sparse_decode_step(sh, w.q_comp, w.k_comp_cache, w.q, w.k_cache, w.v_cache, w.page_table,
                         w.seq_lens, cfg.topk, 0, 0.0, out, idx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(idx), to_np(ref["idx"]))
    np.testing.assert_array_equal(to_np(out.view(torch.int16)), to_np(ref["out"].view(torch.int16)))


@pytest.mark.parametrize("L,hi,heads,topk,values", [(1500, 2, 32, 300, "normal"),
                                                    (900, 4, 16, 128, "int"),
                                                    (2100, 8, 64, 2048, "normal")])
def test_multihead_prefill(L, hi, heads, topk, values):
    cfg = W.small_config(name=f"mh_prefill{hi}", batch=1, lengths=(L,), prefill=True, d_c=64,
                         num_heads=heads, topk=topk, values=values, num_idx_heads=hi)
    w = W.make_workload(cfg, L + hi, device=DEV)
    scores = PL.index_score(w)
    sel = PL.topk_select(w)
    sel_given = PL.topk_select(w, scores=scores)
    out, lse = PL.gather_attend(w, sel["idx"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(sel["idx"]), to_np(sel_given["idx"]))
    wc = W.to_device(w, "cpu")
    rep = check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()}, out,
                         to_np(lse), exact=values == "int")
    say(cfg.name, rep)


def test_multihead_prefill_beyond_the_mask_kernel():
    """258 pages at topk 64: the prefill attention takes the per-row gather."""
    cfg = W.small_config(name="mh_prefill_long", batch=1, lengths=(16500,), prefill=True,
                         d_c=64, num_heads=8, topk=64, num_idx_heads=2)
    w = W.make_workload(cfg, 9, device=DEV)
    assert w.max_pages > 256
    scores = PL.index_score(w)
    sel = PL.topk_select(w, scores=scores)
    out, lse = PL.gather_attend(w, sel["idx"])
    torch.cuda.synchronize()
    wc = W.to_device(w, "cpu")
    say(cfg.name, check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()}, out,
                                 to_np(lse)))


def test_config_multihead_decode_32k_128k():
    """The full-size multi-head workload, every (sequence, indexer head)."""
    w = W.make_workload(W.CONFIGS["multihead_decode_32k_128k"], 0, device=DEV)
    cfg = w.config
    scores = PL.index_score(w)
    sel = PL.topk_select(w)
    step = PL.decode_step(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(step["idx"]), to_np(sel["idx"]))
    wc = W.to_device(w, "cpu")
    rep = check_all_rows(wc, to_np(scores), {k: to_np(v) for k, v in sel.items()}, step["out"],
                         to_np(step["lse"]))
    say(cfg.name, rep)
