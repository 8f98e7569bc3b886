"""Seeded synthetic inputs for index-selected sparse attention.

This module only draws arrays. It holds none of the method's arithmetic: no
scoring, no selection, no attention. The GPU library and the CPU oracle both
consume what it produces, so a test hands the very same arrays to both sides.

The workloads follow the method as the pages state it: compressed query/key
representations (``q_comp``, ``k_comp``) for the indexer, full-width
``q``/``K``/``V`` for the attention, and a KV cache organised in fixed-size
blocks addressed through a page table ("Day-0 Inference Adaptation for
Ultra-Large MoE Models on Domestic GPUs", section "Reorganizing KV Cache
Layout"; "Day-0 Adaptation for Trillion-Parameter MoE Models", section IV).
The pages print no sizes, so the named configurations below are synthetic
stand-ins with the stated shapes and value distributions.

Draw order per workload (fixed, so a seed pins every array). The structure
comes from a seeded CPU ``torch.Generator`` whatever the device, so that the
lengths and page tables (and with them every byte count) are the same on a
host without a GPU: lengths -> page table -> shifted-page choice (block-pruned
config). The values come from a second generator with the same seed on the
target device: q_comp -> k_comp -> K -> V -> q -> per-step stream rows (long
decode stream). Values are drawn as float32 and rounded to bfloat16
(round-to-nearest-even) by ``Tensor.to``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch

BF16 = torch.bfloat16


@dataclass(frozen=True)
class Config:
    """One synthetic workload shape.

    lengths: ("fixed", L) or ("uniform", lo, hi) (integers, inclusive) or
             ("list", (L0, L1, ...)).
    prefill: True -> one query row per context position (q_start = 0);
             False -> one decode query at position L - 1.
    values:  "normal" -> N(0, 1); "int" -> integers uniform in [-3, 3]
             (every product and partial sum of a score is then exact in fp32).
    num_idx_heads: indexer heads Hi; q_comp is then [B, S_q, Hi, d_c] (for
             Hi = 1 it keeps its [B, S_q, d_c] shape, same bytes), and query
             head h attends over the selection of indexer head h // (H / Hi).
    """

    name: str
    batch: int
    lengths: tuple
    prefill: bool
    d_c: int
    num_heads: int
    head_dim: int = 128
    block_size: int = 64
    topk: int = 2048
    n_sel_pages: int = 0
    kcomp_scale: float = 1.0
    shift_frac: float = 0.0
    shift_value: float = 0.0
    stream_steps: int = 0
    values: str = "normal"
    q_scale: float = 1.0
    num_idx_heads: int = 1

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The named workloads. Sizes are stated with each; none come from the pages,
# which print no numbers for this path.
CONFIGS = {
    # 1 query at position 4095 over 4096 tokens; d_c 64; 8 query heads on one
    # KV head; top-256; shuffled page table.
    "decode_4k": Config("decode_4k", 1, ("fixed", 4096), False, 64, 8, topk=256),
    # 8192 query rows over the same 8192-token causal context; 16 heads;
    # top-2048 (all valid positions for rows before 2048).
    "prefill_8k": Config("prefill_8k", 1, ("fixed", 8192), True, 64, 16, topk=2048),
    # 64 sequences, contexts uniform in [32768, 131072]; d_c 128 with k_comp
    # scaled by 1/sqrt(d_c); 32 heads; top-2048.
    "batched_decode_32k_128k": Config(
        "batched_decode_32k_128k", 64, ("uniform", 32768, 131072), False, 128, 32,
        topk=2048, kcomp_scale=1.0 / math.sqrt(128.0)),
    # 8 sequences of 262144 tokens; per-page max -> top 64 pages -> exact
    # top-2048 inside them; a quarter of the pages get k_comp + 0.5.
    "block_pruned_256k": Config(
        "block_pruned_256k", 8, ("fixed", 262144), False, 128, 32, topk=2048,
        n_sel_pages=64, shift_frac=0.25, shift_value=0.5),
    # the batched decode workload's contexts with 4 indexer heads: 32
    # sequences, each (sequence, indexer head) selecting its own top-2048 over
    # the shared compressed keys; 64 query heads, 16 per indexer head.
    "multihead_decode_32k_128k": Config(
        "multihead_decode_32k_128k", 32, ("uniform", 32768, 131072), False, 128, 64,
        topk=2048, kcomp_scale=1.0 / math.sqrt(128.0), num_idx_heads=4),
    # one sequence pre-filled to 1,048,320 tokens; 256 decode steps each append
    # one token, ending at exactly 1,048,576 tokens (16384 pages); 64 heads.
    "long_decode_1m": Config(
        "long_decode_1m", 1, ("fixed", 1048320), False, 128, 64, topk=2048,
        stream_steps=256),
}


@dataclass
class Stream:
    """Rows appended by a decode stream, one token per step and sequence."""

    k_comp_new: torch.Tensor  # bf16 [T, B, d_c]
    k_new: torch.Tensor       # bf16 [T, B, D]
    v_new: torch.Tensor       # bf16 [T, B, D]
    q_comp: torch.Tensor      # bf16 [T, B, 1, d_c]
    q: torch.Tensor           # bf16 [T, B, 1, H, D]


@dataclass
class Workload:
    config: Config
    seed: int
    seq_lens: torch.Tensor      # int32 [B]  tokens in the cache per sequence
    q_start: torch.Tensor       # int32 [B]  position of query row 0
    num_q: int                  # query rows per sequence
    max_pages: int              # page-table row stride
    num_phys_pages: int         # physical page pool size
    page_table: torch.Tensor    # int32 [B, max_pages], -1 past a sequence's pages
    q_comp: torch.Tensor        # bf16 [B, S_q, d_c]
    k_comp_cache: torch.Tensor  # bf16 [P, bs, d_c]
    k_cache: torch.Tensor       # bf16 [P, bs, D]
    v_cache: torch.Tensor       # bf16 [P, bs, D]
    q: torch.Tensor             # bf16 [B, S_q, H, D]
    shifted_pages: Optional[torch.Tensor] = None  # int32 [B, n] logical pages, -1 padded
    stream: Optional[Stream] = None
    extra: dict = field(default_factory=dict)

    @property
    def device(self):
        return self.k_comp_cache.device


def _draw(shape, gen, device, values, scale=1.0):
    if values == "int":
        x = torch.randint(-3, 4, shape, generator=gen, device=device, dtype=torch.int32)
        return x.to(torch.float32)
    if values == "normal":
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        return x
    raise ValueError(f"unknown value distribution {values!r}")


def _draw_lengths(cfg: Config, gen) -> list:
    kind = cfg.lengths[0]
    if kind == "fixed":
        return [int(cfg.lengths[1])] * cfg.batch
    if kind == "uniform":
        lo, hi = int(cfg.lengths[1]), int(cfg.lengths[2])
        t = torch.randint(lo, hi + 1, (cfg.batch,), generator=gen)
        return [int(v) for v in t.tolist()]
    if kind == "list":
        ls = [int(v) for v in cfg.lengths[1]]
        if len(ls) != cfg.batch:
            raise ValueError("length list does not match batch")
        return ls
    raise ValueError(f"unknown length spec {cfg.lengths!r}")


def make_workload(cfg: Config, seed: int = 0, device="cpu") -> Workload:
    """Draw every input array of ``cfg`` from ``seed`` on ``device``."""
    device = torch.device(device)
    sgen = torch.Generator(device="cpu")  # structure: lengths, page table, shifted pages
    sgen.manual_seed(int(seed))
    gen = torch.Generator(device=device)  # values
    gen.manual_seed(int(seed))
    B, bs, d_c, H, D = cfg.batch, cfg.block_size, cfg.d_c, cfg.num_heads, cfg.head_dim

    # 1. lengths
    lens = _draw_lengths(cfg, sgen)
    T = cfg.stream_steps
    caps = [L + T for L in lens]
    n_pages = [max(1, -(-c // bs)) for c in caps]
    max_pages = max(n_pages)
    P = sum(n_pages)

    # 2. page table: one random permutation of the pool, split per sequence
    perm = torch.randperm(P, generator=sgen).to(torch.int32)
    page_table_cpu = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        page_table_cpu[b, : n_pages[b]] = perm[off: off + n_pages[b]]
        off += n_pages[b]
    page_table = page_table_cpu.to(device)

    # 3. shifted pages: exactly n_pages/4 logical pages per sequence, chosen
    #    without replacement (applied to k_comp below)
    shift_rows = None
    if cfg.shift_frac > 0.0:
        shift_rows = []
        for b in range(B):
            n_ctx_pages = -(-lens[b] // bs)
            n_shift = int(n_ctx_pages * cfg.shift_frac)
            choice = torch.randperm(n_ctx_pages, generator=sgen)[:n_shift]
            shift_rows.append(torch.sort(choice).values.to(torch.int32))

    if cfg.prefill:
        S_q = max(lens)
        if any(L != S_q for L in lens):
            raise ValueError("prefill workloads need equal lengths")
        q_start = torch.zeros(B, dtype=torch.int32, device=device)
    else:
        S_q = 1
        q_start = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device=device)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=device)

    # values: q_comp, k_comp (kept in fp32 until the shift is applied), K, V, q
    Hi = cfg.num_idx_heads
    q_comp = _draw((B, S_q, Hi * d_c), gen, device, cfg.values).to(BF16)
    q_comp = q_comp.view(B, S_q, Hi, d_c) if Hi > 1 else q_comp
    k_comp32 = _draw((P, bs, d_c), gen, device, cfg.values, cfg.kcomp_scale)
    k_cache = _draw((P, bs, D), gen, device, cfg.values).to(BF16)
    v_cache = _draw((P, bs, D), gen, device, cfg.values).to(BF16)
    q = _draw((B, S_q, H, D), gen, device, cfg.values, cfg.q_scale).to(BF16)

    # the shift is added to the chosen pages in fp32 before rounding
    shifted = None
    if shift_rows is not None:
        for b, choice in enumerate(shift_rows):
            phys = page_table_cpu[b, choice.long()].long().to(device)
            k_comp32[phys] += cfg.shift_value
        # rows padded with -1 (sequences differ in page count)
        width = max(1, max(int(r.numel()) for r in shift_rows))
        shifted = torch.full((B, width), -1, dtype=torch.int32)
        for b, r in enumerate(shift_rows):
            shifted[b, : r.numel()] = r
        shifted = shifted.to(device)
    k_comp_cache = k_comp32.to(BF16)
    del k_comp32

    # per-step rows of a decode stream
    stream = None
    if T > 0:
        stream = Stream(
            k_comp_new=_draw((T, B, d_c), gen, device, cfg.values, cfg.kcomp_scale).to(BF16),
            k_new=_draw((T, B, D), gen, device, cfg.values).to(BF16),
            v_new=_draw((T, B, D), gen, device, cfg.values).to(BF16),
            q_comp=_draw((T, B, 1, Hi * d_c), gen, device, cfg.values).to(BF16).view(
                (T, B, 1, Hi, d_c) if Hi > 1 else (T, B, 1, d_c)),
            q=_draw((T, B, 1, H, D), gen, device, cfg.values, cfg.q_scale).to(BF16),
        )

    return Workload(cfg, int(seed), seq_lens, q_start, S_q, max_pages, P, page_table,
                    q_comp, k_comp_cache, k_cache, v_cache, q, shifted, stream)


def small_config(name="small", batch=2, lengths=(300, 129), prefill=False, d_c=64,
                 num_heads=16, topk=32, n_sel_pages=0, block_size=64, values="normal",
                 **kw) -> Config:
    """A small workload for tests: explicit per-sequence lengths."""
    return Config(name, batch, ("list", tuple(lengths)), prefill, d_c, num_heads,
                  block_size=block_size, topk=topk, n_sel_pages=n_sel_pages,
                  values=values, **kw)


def logical_rows(cache: torch.Tensor, page_table: torch.Tensor, b: int, length: int):
    """The first ``length`` logical rows of sequence ``b`` as a dense tensor.

    Pure indexing (no arithmetic on values): row j lives in physical page
    ``page_table[b, j // bs]`` at slot ``j % bs``.
    """
    bs = cache.shape[1]
    j = torch.arange(length, device=cache.device)
    pages = page_table[b, (j // bs)].long()
    return cache[pages, j % bs]


def permute_pool(w: Workload, seed: int) -> Workload:
    """Same logical content, physical pages shuffled by a fresh permutation."""
    gen = torch.Generator(device=w.device)
    gen.manual_seed(int(seed))
    P = w.num_phys_pages
    perm = torch.randperm(P, generator=gen, device=w.device)  # old page i -> new perm[i]
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P, device=w.device)
    pt = w.page_table.clone()
    valid = pt >= 0
    pt[valid] = perm[pt[valid].long()].to(torch.int32)
    return replace(w, page_table=pt, k_comp_cache=w.k_comp_cache[inv],
                   k_cache=w.k_cache[inv], v_cache=w.v_cache[inv])


def to_device(w: Workload, device) -> Workload:
    mv = lambda t: None if t is None else t.to(device)
    st = None
    if w.stream is not None:
        s = w.stream
        st = Stream(mv(s.k_comp_new), mv(s.k_new), mv(s.v_new), mv(s.q_comp), mv(s.q))
    return replace(w, seq_lens=mv(w.seq_lens), q_start=mv(w.q_start),
                   page_table=mv(w.page_table), q_comp=mv(w.q_comp),
                   k_comp_cache=mv(w.k_comp_cache), k_cache=mv(w.k_cache),
                   v_cache=mv(w.v_cache), q=mv(w.q), shifted_pages=mv(w.shifted_pages),
                   stream=st)


def as_u16(t: torch.Tensor) -> torch.Tensor:
    """bf16 tensor viewed as its uint16 bit pattern (no value change)."""
    return t.contiguous().view(torch.int16)


# ------------------------------------------------- MXFP4 expert weights

@dataclass(frozen=True)
class Mxfp4Config:
    """A pool of MXFP4 expert weight matrices [rows][cols] and the router's
    picks per layer. Element bytes are uniform (every E2M1 code equally
    likely); E8M0 scale bytes are uniform integers in [scale_lo, scale_hi]."""

    name: str
    num_experts: int
    rows: int
    cols: int
    n_sel: int
    layers: int
    scale_lo: int = 110
    scale_hi: int = 136


MXFP4_CONFIGS = {
    # the gate and up projections of one expert (2 x 2048 rows) over a
    # 7168-wide hidden state, a pool of 64 experts (940 MB of MXFP4), 8 experts
    # picked per layer, 16 layers of picks; scales 2^-17 .. 2^9, so that
    # results below the E4M3 subnormals and above 448 both occur
    "mxfp4_experts_4096x7168": Mxfp4Config("mxfp4_experts_4096x7168", 64, 4096, 7168, 8, 16),
}


@dataclass
class Mxfp4Pool:
    config: Mxfp4Config
    packed: torch.Tensor      # uint8 [E, rows, cols/2]
    scales: torch.Tensor      # uint8 [E, rows, cols/32]
    expert_ids: torch.Tensor  # int32 [layers, n_sel]: distinct picks per layer


def make_mxfp4_pool(cfg: Mxfp4Config, seed: int = 0, device="cpu") -> Mxfp4Pool:
    """Draw the pool and the per-layer picks from ``seed``: the picks from a
    CPU generator (distinct experts per layer), the bytes on ``device``."""
    device = torch.device(device)
    sgen = torch.Generator(device="cpu")
    sgen.manual_seed(int(seed))
    ids = torch.stack([torch.randperm(cfg.num_experts, generator=sgen)[: cfg.n_sel]
                       for _ in range(cfg.layers)]).to(torch.int32)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    E, R, K = cfg.num_experts, cfg.rows, cfg.cols
    packed = torch.randint(0, 256, (E, R, K // 2), generator=gen, device=device,
                           dtype=torch.uint8)
    scales = torch.randint(cfg.scale_lo, cfg.scale_hi + 1, (E, R, K // 32), generator=gen,
                           device=device, dtype=torch.uint8)
    return Mxfp4Pool(cfg, packed, scales, ids.to(device))
