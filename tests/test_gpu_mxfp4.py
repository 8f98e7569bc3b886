"""MXFP4 -> FP8 expert-weight conversion on the GPU against the oracle (needs
an MI355X). Every comparison is bit for bit: the conversion is integer work
on bit patterns ("Day-0 Inference Adaptation for Ultra-Large MoE Models on
Domestic GPUs", section "Handling Low-Precision Expert Weights: Online
Conversion and Workspace Reuse"; "Day-0 Adaptation for Trillion-Parameter
MoE Models", section V)."""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
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
    O.set_threads(min(16, os.cpu_count() or 1))
    yield


def _pack(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _gpu_convert(packed, scales, ids, rows, cols, exp_offset=0, out=None):
    pk = torch.from_numpy(np.ascontiguousarray(packed)).to(DEV)
    sc = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    idt = torch.tensor(np.asarray(ids, np.int32), device=DEV)
    if out is None:
        out = torch.full((idt.numel() * rows * cols,), 0xAB, dtype=torch.uint8, device=DEV)
    T.mxfp4_to_fp8_experts(pk, sc, packed.shape[0], rows, cols, idt, out, exp_offset)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, rows, cols)[: idt.numel()]


@pytest.mark.parametrize("exp_offset", [0, -20, 9, -300, 300])
def test_every_code_and_scale_byte(exp_offset):
    """All 16 codes x all 256 scale bytes (256 rows of 32 elements)."""
    rows, cols = 256, 32
    codes = np.tile(np.repeat(np.arange(16, dtype=np.uint8), 2), (rows, 1))
    packed = _pack(codes)[None]
    scales = np.arange(256, dtype=np.uint8).reshape(1, rows, 1)
    got = _gpu_convert(packed, scales, [0], rows, cols, exp_offset)[0]
    want = O.mxfp4_to_fp8(packed[0], scales[0], rows, cols, exp_offset)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (7, 160), (33, 4096), (129, 7168)])
def test_random_pools_and_ragged_sizes(rows, cols):
    """Random bytes over the whole scale range, matrices smaller than one
    workgroup's span and larger ones with a partial last span; ids with
    repeats and out-of-range entries (those slots stay unwritten)."""
    rng = np.random.default_rng(rows * cols)
    E = 5
    packed = rng.integers(0, 256, (E, rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (E, rows, cols // 32), dtype=np.uint8)
    ids = [4, -1, 0, 4, 5, 2]
    got = _gpu_convert(packed, scales, ids, rows, cols)
    want = O.mxfp4_to_fp8_experts(packed, scales, E, rows, cols, np.array(ids, np.int32),
                                  out=np.full((len(ids), rows, cols), 0xAB, np.uint8))
    np.testing.assert_array_equal(got, want)


def test_full_size_pool_every_layer_through_one_workspace():
    """The 64-expert pool of 4096 x 7168 matrices: all 16 layers' picks of 8
    experts go through one FP8 workspace in turn; after each layer the whole
    workspace (8 x 29.4M bytes) equals the oracle's conversion of that layer's
    experts, so nothing of an earlier layer survives."""
    cfg = W.MXFP4_CONFIGS["mxfp4_experts_4096x7168"]
    pool = W.make_mxfp4_pool(cfg, seed=0, device=DEV)
    ws = PL.Fp8Workspace(cfg.n_sel, cfg.rows, cfg.cols, device=DEV)
    pk = pool.packed.cpu().numpy()
    sc = pool.scales.cpu().numpy()
    ids_all = pool.expert_ids.cpu().numpy()
    for layer in (0, 1, 7, 15):
        view = ws.load(pool.packed, pool.scales, pool.expert_ids[layer])
        torch.cuda.synchronize()
        want = O.mxfp4_to_fp8_experts(pk, sc, cfg.num_experts, cfg.rows, cfg.cols, ids_all[layer])
        np.testing.assert_array_equal(view.cpu().numpy(), want)
        say("layer", layer, "experts", list(ids_all[layer]), "bit-exact")


def test_workspace_reuse_with_fewer_experts_keeps_later_slots():
    """A layer that picks fewer experts writes only its slots: the rest keep
    the previous layer's contents; an exp_offset applies to every element."""
    rng = np.random.default_rng(3)
    E, rows, cols = 6, 40, 256
    packed = rng.integers(0, 256, (E, rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(100, 140, (E, rows, cols // 32), dtype=np.uint8)
    out = torch.empty(4 * rows * cols, dtype=torch.uint8, device=DEV)
    first = _gpu_convert(packed, scales, [1, 2, 3, 5], rows, cols, 0, out)
    _gpu_convert(packed, scales, [0, 4], rows, cols, -8, out)
    second = out.cpu().numpy().reshape(4, rows, cols)
    np.testing.assert_array_equal(second[:2], O.mxfp4_to_fp8_experts(
        packed, scales, E, rows, cols, np.array([0, 4], np.int32), -8))
    np.testing.assert_array_equal(second[2:], first[2:])
    np.testing.assert_array_equal(first, O.mxfp4_to_fp8_experts(
        packed, scales, E, rows, cols, np.array([1, 2, 3, 5], np.int32)))
