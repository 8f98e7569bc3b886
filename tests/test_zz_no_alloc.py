"""The no-allocation decode step against the workspace one (needs an MI355X).

sparse_decode_step_noalloc runs the same kernels as sparse_decode_step with
the library's fixed per-device scratch array in place of a caller workspace;
its outputs must equal the workspace version's bit for bit, also when a call
follows a larger one whose contents the array still holds.
"""
import sys

import numpy as np
import pytest
import torch

from top_index_selection_amd import _lib as T
from top_index_selection_amd import pipeline as PL
from top_index_selection_amd import workloads as W

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
    yield


def _noalloc(w, with_idx=True):
    cfg = w.config
    B, H, D = cfg.batch, cfg.num_heads, cfg.head_dim
    out = torch.full((B, 1, H, D), 7.0, dtype=torch.bfloat16, device=DEV)
    idx = torch.full((B, 1, cfg.topk), -7, dtype=torch.int32, device=DEV) if with_idx else None
    wv = torch.full((B, 1, cfg.topk), 7.0, dtype=torch.float32, device=DEV) if with_idx else None
    lse = torch.full((B, 1, H), 7.0, dtype=torch.float32, device=DEV)
    T.sparse_decode_step_noalloc(PL.shape_of(w), w.q_comp, w.k_comp_cache, w.q, w.k_cache,
                                 w.v_cache, w.page_table, w.seq_lens, cfg.topk, cfg.n_sel_pages,
                                 0.0, out, idx, wv, lse)
    return {"out": out, "idx": idx, "w": wv, "lse": lse}


def _same(a, b, keys):
    for k in keys:
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy(), err_msg=k)


# (name, config): the first is the larger call, whose scratch contents (long
# rows: histograms, candidates, split partials) the later, smaller calls find
CASES = [
    W.small_config(name="noalloc_long", batch=6, lengths=(40000, 1, 12289, 33333, 700, 20000),
                   d_c=128, num_heads=32, topk=2048),
    W.small_config(name="noalloc_short", batch=2, lengths=(4097, 300), d_c=64, num_heads=8,
                   topk=256),
    W.small_config(name="noalloc_pruned", batch=3, lengths=(9000, 64, 30000), d_c=128,
                   num_heads=16, topk=512, n_sel_pages=12),
]


def test_noalloc_decode_matches_workspace_decode_on_successive_calls():
    results = []
    for k, cfg in enumerate(CASES):
        w = W.make_workload(cfg, seed=40 + k, device=DEV)
        need = T.workspace_size(PL.shape_of(w), T.TIS_OP_DECODE_STEP, cfg.topk, cfg.n_sel_pages)
        assert need <= T.NOALLOC_SCRATCH_BYTES
        say("no-alloc decode", cfg.name, "needs", need, "bytes of scratch")
        got = _noalloc(w)
        ref = PL.decode_step(w)
        torch.cuda.synchronize()
        _same(got, ref, ("out", "idx", "w", "lse"))
        results.append((w, ref))
    # again, smallest first, and without an idx output (the array then also
    # holds the index list)
    for w, ref in reversed(results):
        got = _noalloc(w, with_idx=False)
        torch.cuda.synchronize()
        _same(got, ref, ("out", "lse"))
        say("repeat", w.config.name, "ok")
