"""The C ABI on the host (CPU only): the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented codes before it
launches anything (no GPU is touched by these tests)."""
import ctypes as C
import os
import re

import pytest

from top_index_selection_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "tis.h")
FAKE = C.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(\w+)\s*\(", text, flags=re.M)


def test_header_and_binding_agree():
    assert sorted(declared_functions()) == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version():
    assert L.abi_version() == 2


def shape(**kw):
    s = dict(batch=2, num_q=1, d_c=128, num_heads=32, max_pages_per_seq=4, num_phys_pages=8)
    s.update(kw)
    return L.make_shape(**s)


def select(sh, topk=16, n_sel_pages=0, ld=256, ws=FAKE, ws_bytes=1 << 30, idx=FAKE, scores=FAKE):
    return L.lib().sparse_topk_select(C.byref(sh), FAKE, FAKE, scores, ld, FAKE, FAKE, None, topk,
                                      n_sel_pages, idx, None, None, None, ws, ws_bytes, None)


def decode(sh, topk=16, ws_bytes=1 << 30, out=FAKE):
    return L.lib().sparse_decode_step(C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, topk,
                                      0, 0.0, out, None, None, None, FAKE, ws_bytes, None)


def attend(sh, phase=L.TIS_PHASE_DECODE, topk=16, ws_bytes=1 << 30):
    return L.lib().paged_gather_attend(C.byref(sh), phase, FAKE, FAKE, FAKE, FAKE, FAKE, topk, 0.0,
                                       FAKE, None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d_c=96), L.TIS_ERR_UNSUPPORTED),
    (dict(d_c=0), L.TIS_ERR_UNSUPPORTED),
    (dict(num_heads=65), L.TIS_ERR_UNSUPPORTED),
    (dict(num_heads=0), L.TIS_ERR_INVALID_ARG),
    (dict(batch=0), L.TIS_ERR_INVALID_ARG),
    (dict(num_q=0), L.TIS_ERR_INVALID_ARG),
    (dict(max_pages_per_seq=0), L.TIS_ERR_INVALID_ARG),
    (dict(num_phys_pages=0), L.TIS_ERR_INVALID_ARG),
    (dict(batch=70000), L.TIS_ERR_UNSUPPORTED),
])
def test_bad_shapes_are_rejected(kw, code):
    assert select(shape(**kw)) == code
    assert L.last_error() != ""


def test_head_dim_and_block_size_are_fixed():
    sh = shape()
    sh.head_dim = 64
    assert select(sh) == L.TIS_ERR_UNSUPPORTED
    sh = shape()
    sh.block_size = 32
    assert select(sh) == L.TIS_ERR_UNSUPPORTED


def test_null_shape():
    assert L.lib().sparse_topk_select(None, FAKE, FAKE, FAKE, 256, FAKE, FAKE, None, 16, 0, FAKE,
                                      None, None, None, FAKE, 1 << 30, None) == L.TIS_ERR_INVALID_ARG


@pytest.mark.parametrize("topk,nsp,code", [
    (0, 0, L.TIS_ERR_INVALID_ARG), (-3, 0, L.TIS_ERR_INVALID_ARG), (4097, 0, L.TIS_ERR_UNSUPPORTED),
    (16, -1, L.TIS_ERR_INVALID_ARG), (16, 193, L.TIS_ERR_UNSUPPORTED)])
def test_bad_topk_and_pages(topk, nsp, code):
    assert select(shape(), topk=topk, n_sel_pages=nsp) == code


def test_small_ld_scores():
    assert select(shape(), ld=255) == L.TIS_ERR_INVALID_ARG


def test_null_idx():
    assert select(shape(), idx=None) == L.TIS_ERR_INVALID_ARG


def test_workspace_too_small_and_misaligned():
    sh = shape()
    need = L.workspace_size(sh, L.TIS_OP_TOPK_SELECT_GIVEN_SCORES, 16, 0)
    assert select(sh, ws_bytes=need - 1 if need else 0) in (
        L.TIS_ERR_WORKSPACE_TOO_SMALL, L.TIS_ERR_INVALID_ARG) or need == 0
    sh = shape(max_pages_per_seq=1000)  # long rows: the candidate path needs workspace
    need = L.workspace_size(sh, L.TIS_OP_TOPK_SELECT, 16, 0)
    assert need > 0
    assert select(sh, scores=None, ld=0, ws_bytes=need - 1) == L.TIS_ERR_WORKSPACE_TOO_SMALL
    assert "workspace" in L.last_error()
    assert select(sh, scores=None, ld=0, ws=C.c_void_p(0x10010), ws_bytes=need) == \
        L.TIS_ERR_INVALID_ARG


def test_decode_step_rejects_prefill_rows_and_nulls():
    assert decode(shape(num_q=2)) == L.TIS_ERR_INVALID_ARG
    assert decode(shape(), out=None) == L.TIS_ERR_INVALID_ARG
    need = L.workspace_size(shape(), L.TIS_OP_DECODE_STEP, 16, 0)
    assert decode(shape(), ws_bytes=need - 1) == L.TIS_ERR_WORKSPACE_TOO_SMALL


def test_attend_rejects_bad_phase():
    assert attend(shape(), phase=7) == L.TIS_ERR_INVALID_ARG
    assert attend(shape(), topk=0) == L.TIS_ERR_INVALID_ARG


def test_index_score_needs_positions():
    sh = shape()
    rc = L.lib().sparse_index_score(C.byref(sh), FAKE, FAKE, FAKE, None, None, FAKE, 256, None)
    assert rc == L.TIS_ERR_INVALID_ARG


def test_append_needs_pointers():
    sh = shape()
    rc = L.lib().paged_kv_append(C.byref(sh), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == L.TIS_ERR_INVALID_ARG


def test_workspace_sizes_are_aligned_and_grow():
    prev = 0
    for pages in (1, 64, 192, 193, 2048):
        sh = shape(batch=8, max_pages_per_seq=pages, num_phys_pages=8 * pages)
        for op in (L.TIS_OP_TOPK_SELECT, L.TIS_OP_DECODE_STEP, L.TIS_OP_GATHER_ATTEND_DECODE):
            n = L.workspace_size(sh, op, 2048, 0)
            assert n % 256 == 0
        n = L.workspace_size(sh, L.TIS_OP_DECODE_STEP, 2048, 0)
        assert n >= prev
        prev = n
    assert L.workspace_size(shape(), L.TIS_OP_INDEX_SCORE, 16, 0) == 0
    assert L.workspace_size(shape(num_q=8), L.TIS_OP_GATHER_ATTEND_PREFILL, 16, 0) == 0
    with pytest.raises(L.TisError):
        L.workspace_size(shape(num_q=2), L.TIS_OP_DECODE_STEP, 16, 0)


def test_stage_timing_names_and_empty_read():
    names = [L.lib().tis_stage_name(i).decode() for i in range(L.TIS_NUM_STAGES)]
    assert names == ["clear", "score", "hist", "collect", "select", "attend", "combine", "append",
                     "convert"]
    assert L.lib().tis_stage_name(99).decode() == ""
    prev = L.stage_timing_enable(False)
    assert all(v == (0.0, 0) for v in L.stage_timing_read().values())
    L.stage_timing_enable(prev)


# ---- the binding refuses tensors smaller than the shape implies, before any
# call into the library (CPU tensors: the size check comes first, so no GPU is
# needed and nothing is launched)

def _t(n, dtype):
    import torch
    return torch.zeros(n, dtype=dtype)


def _full_args():
    import torch
    sh = L.make_shape(batch=2, num_q=1, d_c=64, num_heads=8, max_pages_per_seq=4, num_phys_pages=8)
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    slots = 8 * 64
    return sh, dict(
        q_comp=_t(2 * 64, bf), k_comp_cache=_t(slots * 64, bf), k_cache=_t(slots * 128, bf),
        v_cache=_t(slots * 128, bf), q=_t(2 * 8 * 128, bf), page_table=_t(2 * 4, i32),
        seq_lens=_t(2, i32), q_start=_t(2, i32), scores=torch.zeros(2, 1, 256, dtype=f32),
        idx=_t(2 * 16, i32), w=_t(2 * 16, f32), count=_t(2, i32),
        page_mask=_t(2 * 4, torch.int64), out=_t(2 * 8 * 128, bf), lse=_t(2 * 8, f32))


def _shrunk(a, name):
    import torch
    t = a[name]
    if name == "scores":
        return torch.zeros(1, 1, 256, dtype=t.dtype)
    return t[: t.numel() - 1]


@pytest.mark.parametrize("name", ["q_comp", "k_comp_cache", "page_table", "seq_lens", "q_start",
                                  "scores"])
def test_index_score_refuses_small_tensors(name):
    sh, a = _full_args()
    a[name] = _shrunk(a, name)
    with pytest.raises(ValueError, match=name):
        L.sparse_index_score(sh, a["q_comp"], a["k_comp_cache"], a["page_table"], a["seq_lens"],
                             a["q_start"], a["scores"])


@pytest.mark.parametrize("name", ["q_comp", "k_comp_cache", "page_table", "seq_lens", "idx", "w",
                                  "count", "page_mask"])
def test_topk_select_refuses_small_tensors(name):
    sh, a = _full_args()
    a[name] = _shrunk(a, name)
    with pytest.raises(ValueError, match=name):
        L.sparse_topk_select(sh, a["q_comp"], a["k_comp_cache"], None, a["page_table"],
                             a["seq_lens"], None, 16, 0, a["idx"], a["w"], a["count"],
                             a["page_mask"])


def test_topk_select_refuses_short_score_rows():
    import torch
    sh, a = _full_args()
    with pytest.raises(ValueError, match="scores"):
        L.sparse_topk_select(sh, None, None, torch.zeros(2, 1, 255), a["page_table"],
                             a["seq_lens"], None, 16, 0, a["idx"])


@pytest.mark.parametrize("name", ["q", "k_cache", "v_cache", "page_table", "idx", "out", "lse"])
def test_gather_attend_refuses_small_tensors(name):
    sh, a = _full_args()
    a[name] = _shrunk(a, name)
    with pytest.raises(ValueError, match=name):
        L.paged_gather_attend(sh, L.TIS_PHASE_DECODE, a["q"], a["k_cache"], a["v_cache"],
                              a["page_table"], a["idx"].reshape(2, 1, -1) if name != "idx"
                              else a["idx"], 16, 0.0, a["out"], a["lse"])


def test_gather_attend_refuses_topk_beyond_idx_rows():
    sh, a = _full_args()
    with pytest.raises(ValueError, match="topk"):
        L.paged_gather_attend(sh, L.TIS_PHASE_DECODE, a["q"], a["k_cache"], a["v_cache"],
                              a["page_table"], _t(4 * 16, a["idx"].dtype).reshape(4, 1, 16), 17,
                              0.0, a["out"])


@pytest.mark.parametrize("name", ["q_comp", "q", "k_comp_cache", "k_cache", "v_cache",
                                  "page_table", "seq_lens", "out", "idx", "w", "lse"])
def test_decode_step_refuses_small_tensors(name):
    sh, a = _full_args()
    a[name] = _shrunk(a, name)
    with pytest.raises(ValueError, match=name):
        L.sparse_decode_step(sh, a["q_comp"], a["k_comp_cache"], a["q"], a["k_cache"],
                             a["v_cache"], a["page_table"], a["seq_lens"], 16, 0, 0.0, a["out"],
                             a["idx"], a["w"], a["lse"])


@pytest.mark.parametrize("name", ["k_comp_new", "k_new", "v_new", "k_comp_cache", "page_table"])
def test_append_refuses_small_tensors(name):
    import torch
    sh, a = _full_args()
    a["k_comp_new"] = _t(2 * 64, torch.bfloat16)
    a["k_new"] = _t(2 * 128, torch.bfloat16)
    a["v_new"] = _t(2 * 128, torch.bfloat16)
    a[name] = _shrunk(a, name)
    with pytest.raises(ValueError, match=name):
        L.paged_kv_append(sh, a["k_comp_new"], a["k_new"], a["v_new"], a["page_table"],
                          a["seq_lens"], a["k_comp_cache"], a["k_cache"], a["v_cache"])


def test_noalloc_decode_refuses_shapes_beyond_its_scratch():
    """The no-allocation decode step holds 64 MiB of scratch: a shape that needs
    more is refused with TIS_ERR_UNSUPPORTED before any device call."""
    sh = shape(batch=64, max_pages_per_seq=2048, num_phys_pages=64 * 2048)
    need = L.workspace_size(sh, L.TIS_OP_DECODE_STEP, 2048, 0)
    assert need > L.NOALLOC_SCRATCH_BYTES
    rc = L.lib().sparse_decode_step_noalloc(C.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            2048, 0, 0.0, FAKE, None, None, None, None)
    assert rc == L.TIS_ERR_UNSUPPORTED
    assert "scratch" in L.last_error()
    rc = L.lib().sparse_decode_step_noalloc(C.byref(shape(num_q=2)), FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, 16, 0, 0.0, FAKE, None, None, None, None)
    assert rc == L.TIS_ERR_INVALID_ARG


@pytest.mark.parametrize("hi,heads,code", [(-1, 32, L.TIS_ERR_INVALID_ARG),
                                           (17, 34, L.TIS_ERR_UNSUPPORTED),
                                           (3, 32, L.TIS_ERR_UNSUPPORTED)])
def test_bad_indexer_head_counts(hi, heads, code):
    sh = shape(num_heads=heads)
    sh.num_idx_heads = hi
    assert select(sh) == code
    assert "num_idx_heads" in L.last_error()


def test_indexer_heads_scale_the_selection_workspace():
    one = shape(batch=4, max_pages_per_seq=300, num_phys_pages=1200)
    four = shape(batch=4, max_pages_per_seq=300, num_phys_pages=1200)
    four.num_idx_heads = 4
    zero = shape(batch=4, max_pages_per_seq=300, num_phys_pages=1200)
    zero.num_idx_heads = 0
    n1 = L.workspace_size(one, L.TIS_OP_TOPK_SELECT, 2048, 0)
    assert L.workspace_size(zero, L.TIS_OP_TOPK_SELECT, 2048, 0) == n1
    assert L.workspace_size(four, L.TIS_OP_TOPK_SELECT, 2048, 0) >= 4 * n1 - 4 * 256 * 8
