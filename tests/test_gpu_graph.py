"""The library's calls under HIP graph capture.

A decode step or a prefill selection + attention enqueues only kernel launches
on the caller's stream (no allocation, no memset, no host synchronisation), so
a caller can capture it once into a HIP graph and replay it. Each test captures
through torch's graph capture, replays several times with the program's own
eager work and synchronisations between the replays, and checks every replay
against the eager result bit for bit.
"""
import pytest
import torch

from top_index_selection_amd import _lib as T
from top_index_selection_amd import pipeline as PL
from top_index_selection_amd import workloads as W

pytestmark = pytest.mark.gpu

BITS = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.int32: torch.int32}


def say(*a):
    print(*a, flush=True)


def equal_bits(a, b):
    return torch.equal(a.view(BITS[a.dtype]), b.view(BITS[b.dtype]))


def capture(fn):
    """Warm fn up on a side stream (as torch's capture asks), then capture it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def decode_workload(seed):
    # long rows (clear, histogramming scan, collect, candidate select), a short
    # one and a ragged tail, and split attention with its merge
    cfg = W.small_config(name="graph_decode", batch=4, lengths=(5000, 13000, 40000, 70001),
                         d_c=128, num_heads=32, topk=2048)
    return W.make_workload(cfg, seed, device="cuda")


def test_decode_step_replays_under_a_hip_graph():
    w = decode_workload(seed=4)
    ws = torch.empty(T.workspace_size(PL.shape_of(w), T.TIS_OP_DECODE_STEP, w.config.topk, 0),
                     dtype=torch.uint8, device="cuda")
    ref = PL.decode_step(w, workspace=ws)
    ref = {k: v.clone() for k, v in ref.items()}
    outs = {k: torch.empty_like(v) for k, v in ref.items()}
    say("graph: capture the decode step")
    g = capture(lambda: PL.decode_step(w, workspace=ws, outputs=outs))
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"graph: replay {rep}")
        for k in ref:
            assert equal_bits(outs[k], ref[k]), (rep, k)
        # eager work on the same buffers between replays
        PL.decode_step(w, workspace=ws)
        torch.cuda.synchronize()


def test_decode_graph_reads_the_current_inputs():
    """A replay reads whatever the captured buffers hold at replay time: new
    queries written in place give the eager results for those queries."""
    w = decode_workload(seed=5)
    ws = torch.empty(T.workspace_size(PL.shape_of(w), T.TIS_OP_DECODE_STEP, w.config.topk, 0),
                     dtype=torch.uint8, device="cuda")
    outs = {k: torch.empty_like(v) for k, v in PL.decode_step(w, workspace=ws).items()}
    g = capture(lambda: PL.decode_step(w, workspace=ws, outputs=outs))
    gen = torch.Generator(device="cuda")
    for rep in range(3):
        gen.manual_seed(100 + rep)
        w.q_comp.copy_(torch.randn(w.q_comp.shape, generator=gen, device="cuda").to(torch.bfloat16))
        w.q.copy_(torch.randn(w.q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        torch.cuda.synchronize()
        ref = {k: v.clone() for k, v in PL.decode_step(w, workspace=ws).items()}
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"graph: replay {rep} on new queries")
        for k in ref:
            assert equal_bits(outs[k], ref[k]), (rep, k)


def test_prefill_select_and_attention_replay_under_a_hip_graph():
    cfg = W.small_config(name="graph_prefill", batch=2, lengths=(3000, 3000), prefill=True,
                         d_c=64, num_heads=16, topk=512)
    w = W.make_workload(cfg, 6, device="cuda")
    sh = PL.shape_of(w)
    ws = torch.empty(T.workspace_size(sh, T.TIS_OP_TOPK_SELECT, cfg.topk, 0), dtype=torch.uint8,
                     device="cuda")
    idx = torch.empty((cfg.batch, w.num_q, cfg.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((cfg.batch, w.num_q, cfg.num_heads, cfg.head_dim), dtype=torch.bfloat16,
                      device="cuda")

    def step():
        T.sparse_topk_select(sh, w.q_comp, w.k_comp_cache, None, w.page_table, w.seq_lens,
                             w.q_start, cfg.topk, 0, idx, workspace=ws)
        T.paged_gather_attend(sh, T.TIS_PHASE_PREFILL, w.q, w.k_cache, w.v_cache, w.page_table,
                              idx, cfg.topk, 0.0, out)

    step()
    torch.cuda.synchronize()
    ref_idx, ref_out = idx.clone(), out.clone()
    g = capture(step)
    for rep in range(3):
        idx.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"graph: prefill replay {rep}")
        assert torch.equal(idx, ref_idx), rep
        assert equal_bits(out, ref_out), rep
        step()
        torch.cuda.synchronize()


def test_no_allocation_step_replays_under_a_hip_graph():
    """The entry point for callers that cannot allocate, captured after a first
    eager call (which takes the scratch array's device address)."""
    w = decode_workload(seed=7)
    cfg = w.config
    ref = PL.decode_step(w)
    ref = {k: v.clone() for k, v in ref.items()}
    outs = {k: torch.empty_like(v) for k, v in ref.items()}
    sh = PL.shape_of(w)

    def step():
        T.sparse_decode_step_noalloc(sh, w.q_comp, w.k_comp_cache, w.q, w.k_cache, w.v_cache,
                                     w.page_table, w.seq_lens, cfg.topk, 0, 0.0, outs["out"],
                                     outs["idx"], outs["w"], outs["lse"])

    step()
    torch.cuda.synchronize()
    g = capture(step)
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"graph: no-allocation replay {rep}")
        for k in ref:
            assert equal_bits(outs[k], ref[k]), (rep, k)
        step()
        torch.cuda.synchronize()
