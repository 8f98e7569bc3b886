"""Pins of the CPU oracle against things other than itself (CPU only).

Each test fixes part of what the oracle computes with an independent route:
exact integer arithmetic, a brute-force rank count, Python/numpy/torch library
routines on the unpaged (logical) arrays, closed forms of attention, the
page-selection invariants, and a hand-worked example in tests/golden.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import oracle as O
from top_index_selection_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _logical(cache, w, b, n):
    return W.logical_rows(cache, w.page_table, b, n)


def _positions(w):
    return [[int(w.q_start[b]) + i for i in range(w.num_q)] for b in range(w.config.batch)]


def _rank_select(s, p, topk):
    """Brute force: j is selected iff fewer than K' candidates outrank it."""
    n = p + 1
    k = min(topk, n)
    chosen = []
    for j in range(n):
        rank = sum(1 for i in range(n) if s[i] > s[j] or (s[i] == s[j] and i < j))
        if rank < k:
            chosen.append(j)
    return chosen


# ------------------------------------------------------------------ scoring

@pytest.mark.parametrize("d_c", [64, 128])
def test_scores_exact_on_integer_inputs(oracle_lib, d_c):
    cfg = W.small_config(lengths=(300, 129), d_c=d_c, values="int", topk=16)
    w = W.make_workload(cfg, seed=3)
    sh = O.shape_of(w)
    sc = O.index_scores(sh, w.q_comp, w.k_comp_cache, w.page_table, w.seq_lens, w.q_start)
    for b, pos in enumerate(_positions(w)):
        for i, p in enumerate(pos):
            kc = _logical(w.k_comp_cache, w, b, p + 1).to(torch.int64)
            qc = w.q_comp[b, i].to(torch.int64)
            exact = (kc @ qc).numpy().astype(np.float32)
            np.testing.assert_array_equal(sc[b, i, : p + 1], exact)
            assert np.isnan(sc[b, i, p + 1:]).all(), "positions after the query must stay untouched"


def test_scores_normal_match_float64_matmul(oracle_lib):
    cfg = W.small_config(lengths=(257, 64, 1), d_c=128, batch=3, topk=8)
    w = W.make_workload(cfg, seed=11)
    sh = O.shape_of(w)
    sc = O.index_scores(sh, w.q_comp, w.k_comp_cache, w.page_table, w.seq_lens, w.q_start)
    for b, pos in enumerate(_positions(w)):
        p = pos[0]
        kc = _logical(w.k_comp_cache, w, b, p + 1).to(torch.float64).numpy()
        qc = w.q_comp[b, 0].to(torch.float64).numpy()
        ref = (kc @ qc).astype(np.float32)
        got = sc[b, 0, : p + 1]
        ulp = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1
        assert (ulp == 0).mean() > 0.95


def test_scores_prefill_rows_are_causal(oracle_lib):
    cfg = W.small_config(lengths=(96,), batch=1, prefill=True, d_c=64, values="int", topk=8)
    w = W.make_workload(cfg, seed=5)
    sh = O.shape_of(w)
    sc = O.index_scores(sh, w.q_comp, w.k_comp_cache, w.page_table, w.seq_lens, w.q_start)
    kc = _logical(w.k_comp_cache, w, 0, 96).to(torch.int64)
    full = (w.q_comp[0].to(torch.int64) @ kc.T).numpy().astype(np.float32)
    for i in range(96):
        np.testing.assert_array_equal(sc[0, i, : i + 1], full[i, : i + 1])
        assert np.isnan(sc[0, i, i + 1:]).all()


# ---------------------------------------------------------------- selection

def _select_rows(scores_rows, positions, topk, block_size=64, n_sel_pages=0):
    """Run the oracle's selection on explicit score rows (batch 1, S_q rows)."""
    S = len(positions)
    ld = scores_rows.shape[-1]
    max_pages = -(-ld // block_size)
    sh = O.shape(1, S, 1, 1, 1, block_size, max_pages)
    sc = np.zeros((1, S, max_pages * block_size), np.float32)
    sc[0, :, :ld] = scores_rows
    return O.topk_select(sh, sc, None, np.array([positions[0]], np.int32), topk, n_sel_pages)


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 300), levels=st.sampled_from([3, 7, 1000]), extra=st.integers(0, 5),
       frac=st.floats(0.0, 1.2), seed=st.integers(0, 2**31 - 1))
def test_topk_matches_bruteforce_rank(oracle_lib, n, levels, extra, frac, seed):
    rng = np.random.default_rng(seed)
    s = (rng.integers(0, levels, size=n) - levels // 2).astype(np.float32)
    p = n - 1
    topk = max(1, min(int(frac * n) + extra, n + 5))
    res = _select_rows(s[None, :], [p], topk)
    want = _rank_select(s, p, topk)
    k = len(want)
    assert res["count"][0, 0] == k
    np.testing.assert_array_equal(res["idx"][0, 0, :k], want)
    assert (res["idx"][0, 0, k:] == -1).all()
    np.testing.assert_array_equal(res["w"][0, 0, :k], s[want])


def test_topk_matches_python_sorted_over_rows(oracle_lib):
    rng = np.random.default_rng(7)
    L = 200
    s = np.round(rng.standard_normal((L, L)) * 4).astype(np.float32) / 4  # many exact ties
    positions = list(range(L))
    sh = O.shape(1, L, 1, 1, 1, 16, -(-L // 16))
    sc = np.zeros((1, L, sh.max_pages * 16), np.float32)
    sc[0, :, :L] = s
    for topk in (1, 5, 37, 64, 250):
        res = O.topk_select(sh, sc, None, np.array([0], np.int32), topk)
        for i in positions:
            order = sorted(range(i + 1), key=lambda j: (-s[i, j], j))
            want = sorted(order[:topk])
            k = len(want)
            assert res["count"][0, i] == k
            np.testing.assert_array_equal(res["idx"][0, i, :k], want)


def test_topk_one_is_first_argmax(oracle_lib):
    rng = np.random.default_rng(1)
    for _ in range(50):
        n = int(rng.integers(1, 500))
        s = rng.integers(-5, 5, size=n).astype(np.float32)
        res = _select_rows(s[None, :], [n - 1], 1)
        assert res["idx"][0, 0, 0] == int(np.argmax(s))


def test_topk_at_least_context_takes_everything(oracle_lib):
    rng = np.random.default_rng(2)
    s = rng.standard_normal(130).astype(np.float32)
    for p in (0, 1, 63, 64, 129):
        res = _select_rows(s[None, :], [p], 200)
        assert res["count"][0, 0] == p + 1
        np.testing.assert_array_equal(res["idx"][0, 0, : p + 1], np.arange(p + 1))
        assert (res["idx"][0, 0, p + 1:] == -1).all()


def test_golden_tie_rule_example(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "tie_rule_example.json")))
    s = np.array(g["scores"], np.float32)
    for case in g["cases"]:
        bs = case["block_size"]
        res = _select_rows(s[None, :], [case["p"]], case["topk"], bs, case["n_sel_pages"])
        np.testing.assert_array_equal(res["idx"][0, 0], case["idx"], err_msg=str(case))
        if "pages" in case:
            np.testing.assert_array_equal(res["sel_pages"][0, 0], case["pages"], err_msg=str(case))
    z = g["signed_zero"]
    res = _select_rows(np.array(z["scores"], np.float32)[None, :], [z["p"]], z["topk"])
    np.testing.assert_array_equal(res["idx"][0, 0], z["idx"])


def test_page_mask_is_a_bijection_with_idx(oracle_lib):
    rng = np.random.default_rng(4)
    L, bs = 333, 64
    s = rng.standard_normal(L).astype(np.float32)
    res = _select_rows(s[None, :], [L - 1], 100, bs)
    mask = res["page_mask"][0, 0]
    bits = sorted(g * bs + t for g in range(mask.size) for t in range(bs)
                  if (int(mask[g]) >> t) & 1)
    k = res["count"][0, 0]
    assert sum(bin(int(m)).count("1") for m in mask) == k
    np.testing.assert_array_equal(bits, res["idx"][0, 0, :k])


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 300), bs=st.sampled_from([4, 16, 64]), n_sel=st.integers(1, 8),
       topk=st.integers(1, 305), levels=st.sampled_from([4, 1000]), seed=st.integers(0, 2**31 - 1))
def test_block_pruned_invariants(oracle_lib, n, bs, n_sel, topk, levels, seed):
    rng = np.random.default_rng(seed)
    s = (rng.integers(0, levels, size=n) - levels // 2).astype(np.float32)
    p = n - 1
    res = _select_rows(s[None, :], [p], topk, bs, n_sel)
    n_pg = p // bs + 1
    maxima = [float(s[g * bs: min(g * bs + bs, n)].max()) for g in range(n_pg)]
    # the kept pages are exactly the brute-force top pages by (max desc, page asc)
    page_rank = [sum(1 for h in range(n_pg) if maxima[h] > maxima[g] or
                     (maxima[h] == maxima[g] and h < g)) for g in range(n_pg)]
    want_pages = [g for g in range(n_pg) if page_rank[g] < min(n_sel, n_pg)]
    got_pages = [g for g in res["sel_pages"][0, 0] if g >= 0]
    assert got_pages == want_pages
    # every selected position lies in a kept page and at or before the query
    k = int(res["count"][0, 0])
    sel = res["idx"][0, 0, :k]
    assert all(j <= p and (j // bs) in want_pages for j in sel)
    # exactly the brute-force top-k among the kept pages' positions
    cand = [j for j in range(n) if (j // bs) in want_pages]
    sub = np.array([s[j] for j in cand], np.float32)
    ranked = [cand[t] for t in _rank_select(sub, len(cand) - 1, topk)]
    np.testing.assert_array_equal(sel, sorted(ranked))
    # pruning cannot lose a top-k position once the kept pages number >= topk
    # (or every page is kept)
    if n_sel >= topk or n_sel >= n_pg:
        exact = _select_rows(s[None, :], [p], topk, bs, 0)
        np.testing.assert_array_equal(res["idx"], exact["idx"])


def test_block_pruned_uses_logical_page_order_on_ties(oracle_lib):
    # four pages with equal maxima: the lowest logical pages are kept
    bs = 16
    s = np.zeros(64, np.float32)
    s[[3, 20, 40, 63]] = 9.0
    res = _select_rows(s[None, :], [63], 2, bs, 2)
    assert list(res["sel_pages"][0, 0]) == [0, 1]
    assert list(res["idx"][0, 0]) == [3, 20]


# ---------------------------------------------------------------- attention

def _sdpa_rows(w, b, i, p, scale):
    """torch's scaled-dot-product attention in fp64 over positions 0..p."""
    k = _logical(w.k_cache, w, b, p + 1).to(torch.float64)
    v = _logical(w.v_cache, w, b, p + 1).to(torch.float64)
    q = w.q[b, i].to(torch.float64)  # [H, D]
    out = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], k[None].expand(q.shape[0], -1, -1), v[None].expand(q.shape[0], -1, -1),
        scale=scale)[:, 0]
    lse = torch.logsumexp(scale * (q @ k.T), dim=-1)
    return out.numpy(), lse.numpy()


def test_attend_equals_dense_causal_when_topk_covers_context(oracle_lib):
    cfg = W.small_config(lengths=(150, 64, 1), batch=3, d_c=64, num_heads=5, topk=160)
    w = W.make_workload(cfg, seed=21)
    sh = O.shape_of(w)
    res = O.run(w)
    dense, dense_lse = O.dense_causal_attention(sh, w.q, w.k_cache, w.v_cache, w.page_table,
                                                w.seq_lens, w.q_start)
    scale = 1.0 / math.sqrt(128)
    for b, pos in enumerate(_positions(w)):
        p = pos[0]
        ref, ref_lse = _sdpa_rows(w, b, 0, p, scale)
        np.testing.assert_allclose(res["out"][b, 0], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"][b, 0], ref_lse, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dense[b, 0], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dense_lse[b, 0], ref_lse, rtol=1e-12, atol=1e-12)


def test_dense_causal_prefill_matches_sdpa(oracle_lib):
    cfg = W.small_config(lengths=(80,), batch=1, prefill=True, d_c=64, num_heads=3, topk=8)
    w = W.make_workload(cfg, seed=8)
    sh = O.shape_of(w)
    dense, _ = O.dense_causal_attention(sh, w.q, w.k_cache, w.v_cache, w.page_table,
                                        w.seq_lens, w.q_start)
    for i in (0, 1, 17, 79):
        ref, _ = _sdpa_rows(w, 0, i, i, 1.0 / math.sqrt(128))
        np.testing.assert_allclose(dense[0, i], ref, rtol=1e-12, atol=1e-12)


def test_attend_closed_forms(oracle_lib):
    cfg = W.small_config(lengths=(200,), batch=1, d_c=64, num_heads=4, topk=12)
    w = W.make_workload(cfg, seed=9)
    sh = O.shape_of(w)
    res = O.run(w, want_probs=True)
    # softmax weights over the selected set sum to one
    assert np.abs(res["probs"].sum(-1) - 1.0).max() < 1e-6
    idx = res["idx"]
    # one selected position: the output is that V row exactly
    one = np.full_like(idx, -1)
    one[..., 0] = idx[..., 3]
    out, lse = O.attend(sh, w.q, w.k_cache, w.v_cache, w.page_table, one)
    v_row = _logical(w.v_cache, w, 0, 200)[int(idx[0, 0, 3])].to(torch.float64).numpy()
    for h in range(4):
        np.testing.assert_array_equal(out[0, 0, h], v_row)
    # constant V: the output is that constant
    vc = torch.full_like(w.v_cache, 0.375)
    out, _ = O.attend(sh, w.q, w.k_cache, vc, w.page_table, idx)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-15)
    # q = 0: the plain mean of the selected V rows, and lse = log K'
    qz = torch.zeros_like(w.q)
    out, lse = O.attend(sh, qz, w.k_cache, w.v_cache, w.page_table, idx)
    sel = idx[0, 0][idx[0, 0] >= 0]
    vv = _logical(w.v_cache, w, 0, 200).to(torch.float64).numpy()[sel]
    for h in range(4):
        np.testing.assert_allclose(out[0, 0, h], vv.mean(0), rtol=1e-12, atol=1e-14)
        assert abs(lse[0, 0, h] - math.log(len(sel))) < 1e-12
    # an empty selection gives zeros and lse = -inf
    none = np.full_like(idx, -1)
    out, lse = O.attend(sh, w.q, w.k_cache, w.v_cache, w.page_table, none)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_attend_matches_sdpa_over_selected_set(oracle_lib):
    cfg = W.small_config(lengths=(300,), batch=1, d_c=128, num_heads=6, topk=40)
    w = W.make_workload(cfg, seed=13)
    res = O.run(w)
    sel = res["idx"][0, 0][: res["count"][0, 0]]
    k = _logical(w.k_cache, w, 0, 300).to(torch.float64)[sel]
    v = _logical(w.v_cache, w, 0, 300).to(torch.float64)[sel]
    q = w.q[0, 0].to(torch.float64)
    scale = 1.0 / math.sqrt(128)
    ref = torch.softmax(scale * (q @ k.T), dim=-1) @ v
    np.testing.assert_allclose(res["out"][0, 0], ref.numpy(), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------- paging

def test_physical_page_permutation_changes_nothing(oracle_lib):
    cfg = W.small_config(lengths=(300, 129), d_c=64, num_heads=4, topk=50)
    w = W.make_workload(cfg, seed=17)
    w2 = W.permute_pool(w, seed=99)
    assert not torch.equal(w.page_table, w2.page_table)
    a, b = O.run(w), O.run(w2)
    for key in ("idx", "w", "count", "page_mask", "out", "lse"):
        np.testing.assert_array_equal(a[key], b[key])


def test_row_sampling_equals_full_batch(oracle_lib):
    cfg = W.small_config(lengths=(100, 77), d_c=64, num_heads=2, topk=20, n_sel_pages=1)
    w = W.make_workload(cfg, seed=23)
    full = O.run(w)
    part = O.run(w, rows=[(1, 0), (0, 0)])
    np.testing.assert_array_equal(part["idx"][0], full["idx"][1, 0])
    np.testing.assert_array_equal(part["idx"][1], full["idx"][0, 0])
    np.testing.assert_array_equal(part["out"][0], full["out"][1, 0])


def test_bf16_rounding_matches_torch(oracle_lib):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-8, 8, 10000),
                        [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65504.0, -1e-40]])
    got = O.to_bf16(x)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(got, want.view(np.uint16))


def test_block_pruned_partial_last_page_uses_valid_positions_only(oracle_lib):
    # positions after the query hold large scores; they must not raise the
    # maximum of the query's last, partial page
    s = np.array([3, 3, 3, 3, 0, 0, 0, 0, 1, 9, 9, 9], np.float32)
    res = _select_rows(s[None, :], [8], 1, 4, 1)
    assert list(res["sel_pages"][0, 0]) == [0]
    assert list(res["idx"][0, 0]) == [0]
    res = _select_rows(s[None, :], [8], 2, 4, 2)
    assert list(res["sel_pages"][0, 0]) == [0, 2]
    assert list(res["idx"][0, 0]) == [0, 1]


def test_null_q_start_means_the_last_rows(oracle_lib):
    """Without q_start, query row i of sequence b sits at seq_lens[b] - S_q + i:
    scores, selection and dense attention equal those of the explicit start,
    and the explicit scores equal a numpy matmul over those positions."""
    cfg = W.small_config(lengths=(700, 300), d_c=64, values="int", topk=40)
    w = W.make_workload(cfg, seed=29)
    S = 5
    qc = torch.stack([w.q_comp[:, 0]] * S, dim=1).contiguous()
    qq = torch.stack([w.q[:, 0]] * S, dim=1).contiguous()
    sh = O.shape_of(w, num_q=S)
    start = (w.seq_lens - S).to(torch.int32)
    sc_null = O.index_scores(sh, qc, w.k_comp_cache, w.page_table, w.seq_lens, None)
    sc_expl = O.index_scores(sh, qc, w.k_comp_cache, w.page_table, None, start)
    np.testing.assert_array_equal(sc_null, sc_expl)
    for b in range(cfg.batch):
        L = int(w.seq_lens[b])
        kc = _logical(w.k_comp_cache, w, b, L).to(torch.int64)
        exact = (kc @ qc[b, 0].to(torch.int64)).numpy().astype(np.float32)
        for i in range(S):
            p = L - S + i
            np.testing.assert_array_equal(sc_null[b, i, : p + 1], exact[: p + 1])
    sel_null = O.topk_select(sh, sc_null, w.seq_lens, None, cfg.topk)
    sel_expl = O.topk_select(sh, sc_expl, None, start, cfg.topk)
    for k in ("idx", "w", "count", "page_mask"):
        np.testing.assert_array_equal(sel_null[k], sel_expl[k])
    d_null, l_null = O.dense_causal_attention(sh, qq, w.k_cache, w.v_cache, w.page_table,
                                              w.seq_lens, None)
    d_expl, l_expl = O.dense_causal_attention(sh, qq, w.k_cache, w.v_cache, w.page_table, None,
                                              start)
    np.testing.assert_array_equal(d_null, d_expl)
    np.testing.assert_array_equal(l_null, l_expl)


# ------------------------------------------------------- multi-head indexer
# Scores shaped [B, H, S, S_c] with a top-k along the last axis ("Day-0
# Inference Adaptation of Ultra-Large-Scale MoE Models on Domestic AI
# Accelerators", section 4.1): every (query row, indexer head) selects on its
# own over the shared compressed keys; query head h attends over the set of
# indexer head h // (H / Hi).

def _mh_config(**kw):
    base = dict(name="mh", batch=2, lengths=(300, 129), d_c=64, num_heads=6, topk=16,
                values="int", num_idx_heads=3)
    base.update(kw)
    return W.small_config(**base)


def test_multihead_scores_and_selection_against_bruteforce(oracle_lib):
    """Integer inputs: every head's scores equal an exact integer matmul over
    the logical rows, and every (row, head) selection equals a brute-force
    rank count over that head's scores."""
    cfg = _mh_config()
    w = W.make_workload(cfg, seed=31)
    sh = O.shape_of(w)
    assert sh.num_idx_heads == 3 and tuple(w.q_comp.shape) == (2, 1, 3, 64)
    sc = O.index_scores(sh, w.q_comp, w.k_comp_cache, w.page_table, w.seq_lens, w.q_start)
    sel = O.topk_select(sh, sc, w.seq_lens, w.q_start, cfg.topk)
    assert sc.shape == (2, 1, 3, w.max_pages * 64) and sel["idx"].shape == (2, 1, 3, cfg.topk)
    for b, pos in enumerate(_positions(w)):
        p = pos[0]
        kc = _logical(w.k_comp_cache, w, b, p + 1).to(torch.int64)
        for g in range(3):
            exact = (kc @ w.q_comp[b, 0, g].to(torch.int64)).numpy().astype(np.float32)
            np.testing.assert_array_equal(sc[b, 0, g, : p + 1], exact)
            chosen = _rank_select(exact.tolist(), p, cfg.topk)
            k = len(chosen)
            assert sel["count"][b, 0, g] == k
            assert sel["idx"][b, 0, g, :k].tolist() == chosen
            assert (sel["idx"][b, 0, g, k:] == -1).all()
        # the heads really differ (else the test would not see a head mix-up)
        assert len({tuple(sel["idx"][b, 0, g]) for g in range(3)}) > 1


def test_multihead_prefill_rows_share_their_query_position(oracle_lib):
    """Prefill rows: head g of query row i sits at the row's own position, and
    its selection equals a brute-force rank over its scores."""
    cfg = _mh_config(batch=1, lengths=(200,), prefill=True, num_idx_heads=2, num_heads=4,
                     topk=30)
    w = W.make_workload(cfg, seed=37)
    sh = O.shape_of(w)
    sc = O.index_scores(sh, w.q_comp, w.k_comp_cache, w.page_table, w.seq_lens, w.q_start)
    sel = O.topk_select(sh, sc, w.seq_lens, w.q_start, cfg.topk)
    kc = _logical(w.k_comp_cache, w, 0, 200).to(torch.int64)
    for i in (0, 1, 29, 30, 31, 199):
        for g in range(2):
            exact = (kc[: i + 1] @ w.q_comp[0, i, g].to(torch.int64)).numpy().astype(np.float32)
            np.testing.assert_array_equal(sc[0, i, g, : i + 1], exact)
            assert np.isnan(sc[0, i, g, i + 1:]).all()
            chosen = _rank_select(exact.tolist(), i, cfg.topk)
            assert sel["idx"][0, i, g, : len(chosen)].tolist() == chosen


def test_multihead_attention_groups_match_sdpa(oracle_lib):
    """Query head h attends over the set of indexer head h // (H / Hi): torch
    SDPA in fp64 over that set's gathered K and V rows."""
    cfg = _mh_config(values="normal", num_idx_heads=2, num_heads=6, topk=40,
                     lengths=(500, 260))
    w = W.make_workload(cfg, seed=41)
    sh = O.shape_of(w)
    sc = O.index_scores(sh, w.q_comp, w.k_comp_cache, w.page_table, w.seq_lens, w.q_start)
    sel = O.topk_select(sh, sc, w.seq_lens, w.q_start, cfg.topk)
    out, lse = O.attend(sh, w.q, w.k_cache, w.v_cache, w.page_table, sel["idx"])
    scale = 1.0 / math.sqrt(cfg.head_dim)
    for b in range(cfg.batch):
        L = int(w.seq_lens[b])
        K = _logical(w.k_cache, w, b, L).double()
        V = _logical(w.v_cache, w, b, L).double()
        for h in range(cfg.num_heads):
            g = h // 3
            j = torch.from_numpy(sel["idx"][b, 0, g][sel["idx"][b, 0, g] >= 0].astype(np.int64))
            q = w.q[b, 0, h].double()[None, None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, K[j][None, None], V[j][None, None], scale=scale)[0, 0, 0]
            np.testing.assert_allclose(out[b, 0, h], ref.numpy(), rtol=1e-12, atol=1e-12)
            logits = (K[j] @ w.q[b, 0, h].double()) * scale
            np.testing.assert_allclose(lse[b, 0, h], torch.logsumexp(logits, 0).item(), rtol=1e-12)


def test_one_indexer_head_reduces_to_the_shared_path(oracle_lib):
    """A zero head count reads as one head; and head g of a multi-head problem
    equals the one-head problem whose q_comp is head g's row."""
    cfg = _mh_config(values="normal", num_idx_heads=2, num_heads=4, topk=50)
    w = W.make_workload(cfg, seed=43)
    sh = O.shape_of(w)
    sc = O.index_scores(sh, w.q_comp, w.k_comp_cache, w.page_table, w.seq_lens, w.q_start)
    sel = O.topk_select(sh, sc, w.seq_lens, w.q_start, cfg.topk)
    out, _ = O.attend(sh, w.q, w.k_cache, w.v_cache, w.page_table, sel["idx"])
    for g in range(2):
        sh1 = O.shape(cfg.batch, 1, cfg.d_c, 2, cfg.head_dim, 64, w.max_pages, 0)  # 0 heads: one
        qc = w.q_comp[:, :, g].contiguous()
        sc1 = O.index_scores(sh1, qc, w.k_comp_cache, w.page_table, w.seq_lens, w.q_start)
        np.testing.assert_array_equal(np.nan_to_num(sc1), np.nan_to_num(sc[:, :, g]))
        sel1 = O.topk_select(sh1, sc1, w.seq_lens, w.q_start, cfg.topk)
        np.testing.assert_array_equal(sel1["idx"], sel["idx"][:, :, g])
        out1, _ = O.attend(sh1, w.q[:, :, 2 * g: 2 * g + 2].contiguous(), w.k_cache, w.v_cache,
                           w.page_table, sel1["idx"])
        np.testing.assert_array_equal(out1, out[:, :, 2 * g: 2 * g + 2])
