"""ctypes binding of libtis.so (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch
tensors on the GPU; it checks that every tensor holds at least the elements
the shape implies, checks dtypes, devices and contiguity, passes raw pointers
and the current HIP stream, and raises TisError on a nonzero return.
All computation happens in the HIP kernels of libtis.so; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtis.so")

TIS_OK = 0
TIS_ERR_INVALID_ARG = -1
TIS_ERR_UNSUPPORTED = -2
TIS_ERR_WORKSPACE_TOO_SMALL = -3
TIS_ERR_HIP = -4

TIS_PHASE_DECODE = 0
TIS_PHASE_PREFILL = 1

TIS_OP_INDEX_SCORE = 0
TIS_OP_TOPK_SELECT = 1
TIS_OP_TOPK_SELECT_GIVEN_SCORES = 2
TIS_OP_GATHER_ATTEND_DECODE = 3
TIS_OP_GATHER_ATTEND_PREFILL = 4
TIS_OP_DECODE_STEP = 5

EXPORTS = ("sparse_index_score", "sparse_topk_select", "paged_gather_attend",
           "sparse_decode_step", "paged_kv_append", "sparse_decode_step_noalloc",
           "mxfp4_to_fp8_experts",
           "tis_workspace_size", "tis_last_error", "tis_abi_version", "tis_stage_timing_enable",
           "tis_stage_timing_read", "tis_stage_name")
NOALLOC_SCRATCH_BYTES = 64 << 20
TIS_NUM_STAGES = 9


class TisError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libtis error {code}: {message}")
        self.code = code


class Shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_q", C.c_int32), ("d_c", C.c_int32),
                ("num_heads", C.c_int32), ("head_dim", C.c_int32), ("block_size", C.c_int32),
                ("max_pages_per_seq", C.c_int32), ("num_phys_pages", C.c_int32),
                ("num_idx_heads", C.c_int32)]

    def __repr__(self):
        return "Shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None


def lib():
    """Load libtis.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (__graft_entry__.build() or "
                "python top_index_selection_amd/build.py)")
        L = C.CDLL(LIB_PATH)
        P, SP = C.c_void_p, C.POINTER(Shape)
        I32, I64, SZ = C.c_int32, C.c_int64, C.c_size_t
        L.sparse_index_score.argtypes = [SP, P, P, P, P, P, P, I64, P]
        L.sparse_topk_select.argtypes = [SP, P, P, P, I64, P, P, P, I32, I32, P, P, P, P, P, SZ, P]
        L.paged_gather_attend.argtypes = [SP, I32, P, P, P, P, P, I32, C.c_float, P, P, P, SZ, P]
        L.sparse_decode_step.argtypes = [SP, P, P, P, P, P, P, P, I32, I32, C.c_float, P, P, P, P,
                                         P, SZ, P]
        L.paged_kv_append.argtypes = [SP, P, P, P, P, P, P, P, P, P]
        L.sparse_decode_step_noalloc.argtypes = [SP, P, P, P, P, P, P, P, I32, I32, C.c_float, P,
                                                 P, P, P, P]
        L.mxfp4_to_fp8_experts.argtypes = [P, P, I32, I32, I32, P, I32, I32, P, SZ, P]
        L.tis_workspace_size.argtypes = [SP, I32, I32, I32]
        L.tis_workspace_size.restype = SZ
        L.tis_last_error.argtypes = []
        L.tis_last_error.restype = C.c_char_p
        L.tis_abi_version.argtypes = []
        L.tis_stage_timing_enable.argtypes = [C.c_int]
        L.tis_stage_timing_read.argtypes = [P, P, I32]
        L.tis_stage_name.argtypes = [I32]
        L.tis_stage_name.restype = C.c_char_p
        for name in EXPORTS[:7]:
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def last_error() -> str:
    return lib().tis_last_error().decode()


def abi_version() -> int:
    return int(lib().tis_abi_version())


def stage_timing_enable(on: bool) -> bool:
    return bool(lib().tis_stage_timing_enable(1 if on else 0))


def stage_timing_read() -> dict:
    """{stage name: (total ms, launches)} since the last read; waits for the work."""
    ms = (C.c_double * TIS_NUM_STAGES)()
    n = (C.c_int64 * TIS_NUM_STAGES)()
    _check(lib().tis_stage_timing_read(C.cast(ms, C.c_void_p), C.cast(n, C.c_void_p),
                                       TIS_NUM_STAGES))
    return {lib().tis_stage_name(i).decode(): (ms[i], n[i]) for i in range(TIS_NUM_STAGES)}


def _check(rc: int):
    if rc != TIS_OK:
        raise TisError(rc, last_error())


def make_shape(batch, num_q, d_c, num_heads, max_pages_per_seq, num_phys_pages, head_dim=128,
               block_size=64, num_idx_heads=1) -> Shape:
    return Shape(batch, num_q, d_c, num_heads, head_dim, block_size, max_pages_per_seq,
                 num_phys_pages, num_idx_heads)


def workspace_size(shape: Shape, op: int, topk: int, n_sel_pages: int = 0) -> int:
    n = int(lib().tis_workspace_size(C.byref(shape), op, topk, n_sel_pages))
    if n == 0 and last_error():
        raise TisError(TIS_ERR_INVALID_ARG, last_error())
    return n


def _dev(t: Optional[torch.Tensor], dtype, name, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return C.c_void_p(t.data_ptr())


# the current stream's raw handle without building a torch Stream object
# (about 0.5 us instead of 3 us per call, which matters for short decode steps)
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    """The HIP stream to enqueue on: `stream`'s, else the current device's
    current stream."""
    if stream is not None:
        return C.c_void_p(stream.cuda_stream)
    if _current_raw_stream is not None:
        return C.c_void_p(_current_raw_stream(torch.cuda.current_device()))
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _workspace(ws: Optional[torch.Tensor], nbytes: int, device, stream=None):
    """The caller's workspace, or a temporary one. A temporary workspace is
    freed when the wrapper returns, while the kernels may still run: the
    caching allocator reuses it only after the work on the allocating stream,
    so a workspace for another stream is recorded on that stream too."""
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        if stream is not None:
            ws.record_stream(stream)
    if ws.dtype != torch.uint8 or not ws.is_cuda:
        raise TypeError("workspace must be a uint8 GPU tensor")
    return ws, C.c_void_p(ws.data_ptr()), ws.numel()


def _need(t: Optional[torch.Tensor], n: int, name: str):
    """Every kernel indexes its arrays by the shape's sizes: a tensor holding
    fewer elements would send it past the end of the allocation, so such a
    tensor is refused before anything is launched."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements; the shape needs at least {n}")


def _qrows(shape) -> int:
    """Query rows B * S_q (q, out and lse are per query row and head)."""
    return int(shape.batch) * int(shape.num_q)


def _rows(shape) -> int:
    """Selection rows B * S_q * Hi (q_comp, scores, idx, w, count, page_mask)."""
    return _qrows(shape) * max(1, int(shape.num_idx_heads))


def _need_caches(shape, k_comp_cache=None, k_cache=None, v_cache=None):
    slots = int(shape.num_phys_pages) * int(shape.block_size)
    _need(k_comp_cache, slots * int(shape.d_c), "k_comp_cache")
    _need(k_cache, slots * int(shape.head_dim), "k_cache")
    _need(v_cache, slots * int(shape.head_dim), "v_cache")


def _need_seq(shape, page_table=None, seq_lens=None, q_start=None):
    _need(page_table, int(shape.batch) * int(shape.max_pages_per_seq), "page_table")
    _need(seq_lens, int(shape.batch), "seq_lens")
    _need(q_start, int(shape.batch), "q_start")


def _need_scores(shape, scores):
    if scores is None:
        return
    cap = int(shape.max_pages_per_seq) * int(shape.block_size)
    if scores.dim() < 1 or scores.shape[-1] < cap:
        raise ValueError(f"scores' last dimension must hold max_pages_per_seq * block_size = {cap}")
    _need(scores, _rows(shape) * scores.shape[-1], "scores")


BF16, I32, F32 = torch.bfloat16, torch.int32, torch.float32


def sparse_index_score(shape, q_comp, k_comp_cache, page_table, seq_lens, q_start, scores,
                       stream=None):
    _need(q_comp, _rows(shape) * int(shape.d_c), "q_comp")
    _need_caches(shape, k_comp_cache)
    _need_seq(shape, page_table, seq_lens, q_start)
    if scores is None:
        raise ValueError("scores is required")
    _need_scores(shape, scores)
    _check(lib().sparse_index_score(
        C.byref(shape), _dev(q_comp, BF16, "q_comp"), _dev(k_comp_cache, BF16, "k_comp_cache"),
        _dev(page_table, I32, "page_table"), _dev(seq_lens, I32, "seq_lens", True),
        _dev(q_start, I32, "q_start", True), _dev(scores, F32, "scores"), scores.shape[-1],
        _stream(stream)))
    return scores


def sparse_topk_select(shape, q_comp, k_comp_cache, scores, page_table, seq_lens, q_start, topk,
                       n_sel_pages, idx, w=None, count=None, page_mask=None, workspace=None,
                       stream=None):
    op = TIS_OP_TOPK_SELECT if scores is None else TIS_OP_TOPK_SELECT_GIVEN_SCORES
    rows = _rows(shape)
    if scores is None:
        _need(q_comp, rows * int(shape.d_c), "q_comp")
        _need_caches(shape, k_comp_cache)
    _need_scores(shape, scores)
    _need_seq(shape, page_table, seq_lens, q_start)
    if idx is None:
        raise ValueError("idx is required")
    _need(idx, rows * int(topk), "idx")
    _need(w, rows * int(topk), "w")
    _need(count, rows, "count")
    _need(page_mask, rows * int(shape.max_pages_per_seq), "page_mask")
    ws, wsp, wsn = _workspace(workspace, workspace_size(shape, op, topk, n_sel_pages), idx.device,
                              stream)
    _check(lib().sparse_topk_select(
        C.byref(shape), _dev(q_comp, BF16, "q_comp", True),
        _dev(k_comp_cache, BF16, "k_comp_cache", True), _dev(scores, F32, "scores", True),
        0 if scores is None else scores.shape[-1], _dev(page_table, I32, "page_table", True),
        _dev(seq_lens, I32, "seq_lens", True), _dev(q_start, I32, "q_start", True), topk,
        n_sel_pages, _dev(idx, I32, "idx"), _dev(w, F32, "w", True),
        _dev(count, I32, "count", True), _dev(page_mask, torch.int64, "page_mask", True), wsp,
        wsn, _stream(stream)))
    return idx


def paged_gather_attend(shape, phase, q, k_cache, v_cache, page_table, idx, topk, softmax_scale,
                        out, lse=None, workspace=None, stream=None):
    op = TIS_OP_GATHER_ATTEND_DECODE if phase == TIS_PHASE_DECODE else TIS_OP_GATHER_ATTEND_PREFILL
    rows, qrows = _rows(shape), _qrows(shape)
    hd = int(shape.num_heads) * int(shape.head_dim)
    _need(q, qrows * hd, "q")
    _need_caches(shape, None, k_cache, v_cache)
    _need_seq(shape, page_table)
    _need(idx, rows * int(topk), "idx")
    if idx is not None and idx.dim() >= 1 and idx.shape[-1] < int(topk):
        raise ValueError(f"idx rows hold {idx.shape[-1]} entries, fewer than topk = {int(topk)}")
    if out is None:
        raise ValueError("out is required")
    _need(out, qrows * hd, "out")
    _need(lse, qrows * int(shape.num_heads), "lse")
    ws, wsp, wsn = _workspace(workspace, workspace_size(shape, op, topk, 0), out.device, stream)
    _check(lib().paged_gather_attend(
        C.byref(shape), phase, _dev(q, BF16, "q"), _dev(k_cache, BF16, "k_cache"),
        _dev(v_cache, BF16, "v_cache"), _dev(page_table, I32, "page_table"), _dev(idx, I32, "idx"),
        topk, float(softmax_scale), _dev(out, BF16, "out"), _dev(lse, F32, "lse", True), wsp, wsn,
        _stream(stream)))
    return out


def sparse_decode_step(shape, q_comp, k_comp_cache, q, k_cache, v_cache, page_table, seq_lens,
                       topk, n_sel_pages, softmax_scale, out, idx=None, w=None, lse=None,
                       workspace=None, stream=None):
    rows, qrows = _rows(shape), _qrows(shape)
    hd = int(shape.num_heads) * int(shape.head_dim)
    _need(q_comp, rows * int(shape.d_c), "q_comp")
    _need(q, qrows * hd, "q")
    _need_caches(shape, k_comp_cache, k_cache, v_cache)
    _need_seq(shape, page_table, seq_lens)
    if out is None:
        raise ValueError("out is required")
    _need(out, qrows * hd, "out")
    _need(idx, rows * int(topk), "idx")
    _need(w, rows * int(topk), "w")
    _need(lse, qrows * int(shape.num_heads), "lse")
    ws, wsp, wsn = _workspace(workspace, workspace_size(shape, TIS_OP_DECODE_STEP, topk,
                                                        n_sel_pages), out.device, stream)
    _check(lib().sparse_decode_step(
        C.byref(shape), _dev(q_comp, BF16, "q_comp"), _dev(k_comp_cache, BF16, "k_comp_cache"),
        _dev(q, BF16, "q"), _dev(k_cache, BF16, "k_cache"), _dev(v_cache, BF16, "v_cache"),
        _dev(page_table, I32, "page_table"), _dev(seq_lens, I32, "seq_lens"), topk, n_sel_pages,
        float(softmax_scale), _dev(out, BF16, "out"), _dev(idx, I32, "idx", True),
        _dev(w, F32, "w", True), _dev(lse, F32, "lse", True), wsp, wsn, _stream(stream)))
    return out


def sparse_decode_step_noalloc(shape, q_comp, k_comp_cache, q, k_cache, v_cache, page_table,
                               seq_lens, topk, n_sel_pages, softmax_scale, out, idx=None, w=None,
                               lse=None, stream=None):
    """sparse_decode_step without a workspace: the library's fixed scratch
    array of the current device serves instead (calls on one device must not
    overlap)."""
    rows, qrows = _rows(shape), _qrows(shape)
    hd = int(shape.num_heads) * int(shape.head_dim)
    _need(q_comp, rows * int(shape.d_c), "q_comp")
    _need(q, qrows * hd, "q")
    _need_caches(shape, k_comp_cache, k_cache, v_cache)
    _need_seq(shape, page_table, seq_lens)
    if out is None:
        raise ValueError("out is required")
    _need(out, qrows * hd, "out")
    _need(idx, rows * int(topk), "idx")
    _need(w, rows * int(topk), "w")
    _need(lse, qrows * int(shape.num_heads), "lse")
    _check(lib().sparse_decode_step_noalloc(
        C.byref(shape), _dev(q_comp, BF16, "q_comp"), _dev(k_comp_cache, BF16, "k_comp_cache"),
        _dev(q, BF16, "q"), _dev(k_cache, BF16, "k_cache"), _dev(v_cache, BF16, "v_cache"),
        _dev(page_table, I32, "page_table"), _dev(seq_lens, I32, "seq_lens"), topk, n_sel_pages,
        float(softmax_scale), _dev(out, BF16, "out"), _dev(idx, I32, "idx", True),
        _dev(w, F32, "w", True), _dev(lse, F32, "lse", True), _stream(stream)))
    return out


U8 = torch.uint8


def mxfp4_to_fp8_experts(w_packed, w_scales, num_experts, rows, cols, expert_ids, fp8_out,
                         exp_offset=0, stream=None):
    """Dequantise the MXFP4 weights of the experts in `expert_ids` (int32, on
    the GPU) into slots of `fp8_out` (uint8, n_sel * rows * cols bytes at
    least; E4M3 bit patterns)."""
    E, R, K = int(num_experts), int(rows), int(cols)
    n_sel = 0 if expert_ids is None else int(expert_ids.numel())
    _need(w_packed, E * R * (K // 2), "w_packed")
    _need(w_scales, E * R * (K // 32), "w_scales")
    if fp8_out is None:
        raise ValueError("fp8_out is required")
    _need(fp8_out, n_sel * R * K, "fp8_out")
    _check(lib().mxfp4_to_fp8_experts(
        _dev(w_packed, U8, "w_packed"), _dev(w_scales, U8, "w_scales"), E, R, K,
        _dev(expert_ids, I32, "expert_ids"), n_sel, int(exp_offset), _dev(fp8_out, U8, "fp8_out"),
        fp8_out.numel(), _stream(stream)))
    return fp8_out


def paged_kv_append(shape, k_comp_new, k_new, v_new, page_table, seq_lens, k_comp_cache, k_cache,
                    v_cache, stream=None):
    B = int(shape.batch)
    _need(k_comp_new, B * int(shape.d_c), "k_comp_new")
    _need(k_new, B * int(shape.head_dim), "k_new")
    _need(v_new, B * int(shape.head_dim), "v_new")
    _need_seq(shape, page_table, seq_lens)
    _need_caches(shape, k_comp_cache, k_cache, v_cache)
    _check(lib().paged_kv_append(
        C.byref(shape), _dev(k_comp_new, BF16, "k_comp_new"), _dev(k_new, BF16, "k_new"),
        _dev(v_new, BF16, "v_new"), _dev(page_table, I32, "page_table"),
        _dev(seq_lens, I32, "seq_lens"), _dev(k_comp_cache, BF16, "k_comp_cache"),
        _dev(k_cache, BF16, "k_cache"), _dev(v_cache, BF16, "v_cache"), _stream(stream)))
