"""Seeded synthetic workloads for sparse paged decode attention.

This module only draws inputs.  It holds none of the attention arithmetic: it
does no region-to-page resolution and no masking, and it has no softmax.  The
HIP path and the oracle both consume what it produces.  Index structures come
from ``numpy.random.default_rng(seed)``, so they do not depend on the device.
Bulk tensors (query, cache, gate) come from ``torch.Generator(device)`` seeded
with the same seed.  They are drawn in fp32 and rounded to nearest: to bf16,
or to float8_e4m3fn after division by the per-tensor scale.

The five named workloads follow the decode shapes the pages describe.  Each
row is a (token, KV group) pair, and the G*query_len rows of a request share
one block-table row.  The cache is [pages, G, block, 384] with K then V.  A
row selects a set of distinct region ids that always contains the region of
its own position.  The ids are shuffled, and unused slots hold -1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

HEAD_DIM = 192


@dataclass(frozen=True)
class Workload:
    name: str
    requests: int
    query_len: int
    groups: int
    heads: int
    block: int
    pages_per_req: int
    R: int
    kv: str                      # "bf16" or "fp8"
    pos_lo: int                  # first query token position ~ U[pos_lo, pos_hi]
    pos_hi: int
    live: tuple | None = None    # per-row live-slot count ~ U[lo, hi]; None: R
    inactive_frac: float = 0.0   # round(frac * rows) rows inactive
    inactive_rows: tuple = ()    # explicit inactive rows (overrides frac)
    gated: bool = False
    splits: int | None = None    # None: sda_splits(rows)
    k_scale: float = 0.05
    v_scale: float = 0.04
    region_tokens: int = 0       # 0: one region per page
    seed: int = 0

    @property
    def rows(self) -> int:
        return self.requests * self.query_len * self.groups

    @property
    def tokens(self) -> int:
        return self.requests * self.query_len

    @property
    def total_pages(self) -> int:
        return self.requests * self.pages_per_req

    @property
    def rt(self) -> int:
        return self.region_tokens or self.block

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)


def workload_seed(k: int) -> int:
    return 1000 * k + 7


# The five decode workloads (1-based numbering), and two at 8-token regions.
WORKLOADS = {
    1: Workload("tiny-bf16", requests=4, query_len=1, groups=1, heads=8, block=16,
                pages_per_req=16, R=8, kv="bf16", pos_lo=1, pos_hi=127,
                live=None, inactive_rows=(3,), gated=False, splits=1, seed=workload_seed(1)),
    2: Workload("bf16-gated", requests=64, query_len=1, groups=4, heads=16, block=64,
                pages_per_req=512, R=32, kv="bf16", pos_lo=4096, pos_hi=32767,
                inactive_frac=0.05, gated=True, splits=None, seed=workload_seed(2)),
    3: Workload("fp8-cache", requests=256, query_len=1, groups=2, heads=16, block=64,
                pages_per_req=2048, R=64, kv="fp8", pos_lo=65536, pos_hi=131071,
                gated=False, splits=None, seed=workload_seed(3)),
    4: Workload("multi-token", requests=128, query_len=2, groups=4, heads=8, block=32,
                pages_per_req=512, R=64, kv="bf16", pos_lo=8192, pos_hi=16382,
                live=(8, 64), inactive_frac=0.10, gated=True, splits=None,
                seed=workload_seed(4)),
    5: Workload("large-batch-fp8", requests=1024, query_len=1, groups=4, heads=16, block=64,
                pages_per_req=256, R=32, kv="fp8", pos_lo=8192, pos_hi=16383,
                gated=True, splits=1, seed=workload_seed(5)),
    # The pages' own region granularity (8 tokens, many regions per page) at the
    # bf16-gated shape: 256 slots of 8 tokens = the same 2048 tokens per row.
    6: Workload("bf16-gated-8tok", requests=64, query_len=1, groups=4, heads=16, block=64,
                pages_per_req=512, R=256, kv="bf16", pos_lo=4096, pos_hi=32767,
                inactive_frac=0.05, gated=True, splits=None, region_tokens=8,
                seed=workload_seed(6)),
    # The same at the FP8-cache shape: 512 slots of 8 tokens = 4096 tokens per row.
    7: Workload("fp8-cache-8tok", requests=256, query_len=1, groups=2, heads=16, block=64,
                pages_per_req=2048, R=512, kv="fp8", pos_lo=65536, pos_hi=131071,
                gated=False, splits=None, region_tokens=8, seed=workload_seed(7)),
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity cases)."""
    return replace(w, **kw)


@dataclass
class Indices:
    block_table: np.ndarray      # int32 [requests, pages_per_req]
    positions: np.ndarray        # int32 [rows]
    regions: np.ndarray          # int32 [rows, R]
    active: np.ndarray           # uint8 [rows]


def draw_indices(w: Workload, seed: int | None = None, block_table: np.ndarray | None = None
                 ) -> Indices:
    """Block table (a random permutation of all pages), positions, region
    selections and the active mask."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if block_table is None:
        block_table = rng.permutation(w.total_pages).astype(np.int32).reshape(
            w.requests, w.pages_per_req)
    first = rng.integers(w.pos_lo, w.pos_hi + 1, size=w.requests)
    # row r = (request * query_len + j) * G + g; token j of a request sits at first + j
    req = np.repeat(np.arange(w.requests), w.query_len * w.groups)
    j = np.tile(np.repeat(np.arange(w.query_len), w.groups), w.requests)
    positions = (first[req] + j).astype(np.int32)
    rt = w.rt
    regions = np.full((w.rows, w.R), -1, dtype=np.int32)
    for r in range(w.rows):
        cur = int(positions[r]) // rt           # the region holding the row's own token
        avail = cur + 1
        want = w.R if w.live is None else int(rng.integers(w.live[0], w.live[1] + 1))
        n = min(want, avail, w.R)
        if n <= 0:
            continue
        others = rng.choice(cur, size=n - 1, replace=False) if n > 1 else np.zeros(0, np.int64)
        ids = np.concatenate([others, [cur]]).astype(np.int32)
        rng.shuffle(ids)
        regions[r, :n] = ids
    active = np.ones(w.rows, dtype=np.uint8)
    if w.inactive_rows:
        active[list(w.inactive_rows)] = 0
    elif w.inactive_frac > 0:
        k = int(round(w.inactive_frac * w.rows))
        active[rng.choice(w.rows, size=k, replace=False)] = 0
    return Indices(block_table, positions, regions, active)


@dataclass
class Inputs:
    """Everything one decode call takes, on one device."""
    w: Workload
    query: torch.Tensor          # bf16 [rows, heads, 192]
    cache: torch.Tensor          # bf16 or uint8 (e4m3 bytes) [pages, G, block, 384]
    regions: torch.Tensor        # int32 [rows, R]
    block_table: torch.Tensor    # int32 [requests, pages_per_req]
    positions: torch.Tensor      # int32 [rows]
    active: torch.Tensor         # bool [rows]
    gate: torch.Tensor | None    # bf16 [tokens, G*heads]
    k_scale: torch.Tensor | None  # fp32 [1] (FP8 only)
    v_scale: torch.Tensor | None
    scale: float
    splits: int | None           # None: the library's sda_splits(rows)

    @property
    def fp8(self) -> bool:
        return self.cache.dtype == torch.uint8


def draw_cache(w: Workload, device, seed: int | None = None, pages_per_draw: int = 4096
               ) -> torch.Tensor:
    """bf16 ~ N(0,1), or FP8 e4m3 bytes of RN(N(0,1)/scale) (K: k_scale, V: v_scale).
    Drawn in slices of ``pages_per_draw`` pages to bound temporaries."""
    gen = torch.Generator(device=device)
    gen.manual_seed((w.seed if seed is None else seed) * 2 + 1)
    shape = (w.total_pages, w.groups, w.block, 2 * HEAD_DIM)
    if w.kv == "bf16":
        cache = torch.empty(shape, dtype=torch.bfloat16, device=device)
    else:
        cache = torch.empty(shape, dtype=torch.uint8, device=device)
    for p0 in range(0, w.total_pages, pages_per_draw):
        p1 = min(w.total_pages, p0 + pages_per_draw)
        x = torch.randn((p1 - p0,) + shape[1:], generator=gen, device=device)
        if w.kv == "bf16":
            cache[p0:p1] = x.to(torch.bfloat16)
        else:
            x[..., :HEAD_DIM] /= w.k_scale
            x[..., HEAD_DIM:] /= w.v_scale
            cache[p0:p1] = x.to(torch.float8_e4m3fn).view(torch.uint8)
        del x
    return cache


def make_inputs(w: Workload, device="cpu", seed: int | None = None,
                cache: torch.Tensor | None = None, block_table: np.ndarray | None = None,
                splits: int | None = None) -> Inputs:
    """Draw a full input set.  Pass ``cache``/``block_table`` to draw another
    query/selection set over an existing cache."""
    seed = w.seed if seed is None else seed
    idx = draw_indices(w, seed=seed, block_table=block_table)
    if cache is None:
        cache = draw_cache(w, device, seed=seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 2)
    query = torch.randn((w.rows, w.heads, HEAD_DIM), generator=gen, device=device).to(
        torch.bfloat16)
    gate = None
    if w.gated:
        # N(0, 2): variance 2
        g = torch.randn((w.tokens, w.groups * w.heads), generator=gen, device=device)
        gate = (g * math.sqrt(2.0)).to(torch.bfloat16)
    k_scale = v_scale = None
    if w.kv == "fp8":
        k_scale = torch.tensor([w.k_scale], dtype=torch.float32, device=device)
        v_scale = torch.tensor([w.v_scale], dtype=torch.float32, device=device)
    if splits is None:
        splits = w.splits
    return Inputs(
        w=w, query=query, cache=cache,
        regions=torch.from_numpy(idx.regions).to(device),
        block_table=torch.from_numpy(idx.block_table).to(device),
        positions=torch.from_numpy(idx.positions).to(device),
        active=torch.from_numpy(idx.active.astype(bool)).to(device),
        gate=gate, k_scale=k_scale, v_scale=v_scale, scale=w.scale, splits=splits)


# ---- gated sliding-window decode -------------------------------------------
# The non-DSA layers' decode: a uniform batch of requests*query_len tokens, each
# attending over the last `window` tokens of its request in the same packed
# cache.  The pages leave the window length open; 1024 tokens is used here.

@dataclass(frozen=True)
class SwaWorkload:
    name: str
    requests: int
    query_len: int
    groups: int
    heads: int                   # query heads per KV group
    block: int
    pages_per_req: int
    window: int
    seq_lo: int                  # sequence length ~ U[seq_lo, seq_hi]
    seq_hi: int
    gated: bool = True
    splits: int | None = None    # None: sda_swa_plan(...)
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.requests * self.query_len

    @property
    def rows(self) -> int:
        return self.tokens * self.groups

    @property
    def total_pages(self) -> int:
        return self.requests * self.pages_per_req

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)


SWA_WORKLOADS = {
    # decode, 16 heads per KV group, full 1024-token windows in 8K contexts
    "swa-gated": SwaWorkload("swa-gated", requests=256, query_len=1, groups=4, heads=16,
                             block=64, pages_per_req=128, window=1024, seq_lo=1024,
                             seq_hi=8192, seed=workload_seed(11)),
    # MTP verify: 4 query tokens per request, 4 heads per KV group
    "swa-mtp": SwaWorkload("swa-mtp", requests=128, query_len=4, groups=4, heads=4,
                           block=64, pages_per_req=128, window=1024, seq_lo=4,
                           seq_hi=8192, seed=workload_seed(12)),
}


@dataclass
class SwaInputs:
    w: SwaWorkload
    query: torch.Tensor          # bf16 [tokens, G*heads, 192]
    cache: torch.Tensor          # bf16 [pages, G, block, 384]
    block_table: torch.Tensor    # int32 [requests, pages_per_req]
    seq_lens: torch.Tensor       # int32 [requests]
    gate: torch.Tensor | None    # bf16 [tokens, G*heads]
    scale: float
    splits: int | None


def make_swa_inputs(w: SwaWorkload, device="cpu", seed: int | None = None,
                    cache: torch.Tensor | None = None, seq_lens=None,
                    splits: int | None = None) -> SwaInputs:
    """Block table = random permutation of all pages; seq_lens ~ U[seq_lo,
    seq_hi] (or as given); query, cache ~ N(0,1) bf16; gate ~ N(0,2) bf16."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    table = rng.permutation(w.total_pages).astype(np.int32).reshape(w.requests, w.pages_per_req)
    if seq_lens is None:
        seq_lens = rng.integers(w.seq_lo, w.seq_hi + 1, size=w.requests)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (w.requests,)
    assert int(seq_lens.max(initial=0)) <= w.pages_per_req * w.block
    if cache is None:
        cache = draw_cache(Workload(w.name, requests=w.requests, query_len=w.query_len,
                                    groups=w.groups, heads=w.heads, block=w.block,
                                    pages_per_req=w.pages_per_req, R=0, kv="bf16", pos_lo=0,
                                    pos_hi=0, seed=seed), device, seed=seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 2)
    query = torch.randn((w.tokens, w.groups * w.heads, HEAD_DIM), generator=gen,
                        device=device).to(torch.bfloat16)
    gate = None
    if w.gated:
        g = torch.randn((w.tokens, w.groups * w.heads), generator=gen, device=device)
        gate = (g * math.sqrt(2.0)).to(torch.bfloat16)
    return SwaInputs(w=w, query=query, cache=cache,
                     block_table=torch.from_numpy(table).to(device),
                     seq_lens=torch.from_numpy(seq_lens).to(device), gate=gate, scale=w.scale,
                     splits=w.splits if splits is None else splits)


# ---- region selection -------------------------------------------------------
# Scores of 8-token regions for decode rows: row r's current region is
# position // 8 and its candidates are regions 0 .. position // 8.

@dataclass(frozen=True)
class SelectWorkload:
    name: str
    rows: int
    num_regions: int             # score columns S
    topk: int
    pos_lo: int                  # row position ~ U[pos_lo, pos_hi]
    pos_hi: int
    region_tokens: int = 8
    seed: int = 0


SELECT_WORKLOADS = {
    # the bf16-gated decode batch (64 requests x G 4) over 32K contexts
    "select-decode": SelectWorkload("select-decode", rows=256, num_regions=4096, topk=512,
                                    pos_lo=4096, pos_hi=32767, seed=workload_seed(21)),
    # the large batch (1024 requests x G 4) over 128K contexts
    "select-large": SelectWorkload("select-large", rows=4096, num_regions=16384, topk=512,
                                   pos_lo=65536, pos_hi=131071, seed=workload_seed(22)),
}


@dataclass
class SelectInputs:
    w: SelectWorkload
    scores: torch.Tensor         # fp32 [rows, S]
    current: torch.Tensor        # int32 [rows]
    topk_lengths: torch.Tensor   # int32 [rows]


def make_select_inputs(w: SelectWorkload, device="cpu", seed: int | None = None,
                       dist: str = "normal") -> SelectInputs:
    """scores ~ N(0,1) fp32 ("normal"), or small integers with many ties
    ("ties"); positions ~ U[pos_lo, pos_hi]; current = position // region_tokens,
    topk_lengths = current + 1."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    pos = rng.integers(w.pos_lo, w.pos_hi + 1, size=w.rows)
    cur = (pos // w.region_tokens).astype(np.int32)
    lens = np.minimum(cur + 1, w.num_regions).astype(np.int32)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 2 + 1)
    if dist == "normal":
        scores = torch.randn((w.rows, w.num_regions), generator=gen, device=device)
    else:
        scores = torch.randint(0, 8, (w.rows, w.num_regions), generator=gen,
                               device=device).to(torch.float32)
    return SelectInputs(w=w, scores=scores, current=torch.from_numpy(cur).to(device),
                        topk_lengths=torch.from_numpy(lens).to(device))


# ---- decode indexer logits ---------------------------------------------------
# Rows (token, KV group) with `heads` indexer heads of dim 256 in e4m3, fp32
# head weights, and per-region e4m3 summaries of dim 256 kept per page
# (block // region_tokens regions per page) with an fp32 scale per region.

@dataclass(frozen=True)
class LogitsWorkload:
    name: str
    requests: int
    query_len: int
    groups: int
    heads: int
    block: int
    pages_per_req: int
    pos_lo: int
    pos_hi: int
    region_tokens: int = 8
    seed: int = 0

    @property
    def rows(self) -> int:
        return self.requests * self.query_len * self.groups

    @property
    def rpb(self) -> int:
        return self.block // self.region_tokens

    @property
    def num_regions(self) -> int:
        return self.pages_per_req * self.rpb

    @property
    def total_pages(self) -> int:
        return self.requests * self.pages_per_req


LOGITS_WORKLOADS = {
    # the bf16-gated decode batch (64 requests x G 4) over 32K contexts
    "logits-decode": LogitsWorkload("logits-decode", requests=64, query_len=1, groups=4, heads=8,
                                    block=64, pages_per_req=512, pos_lo=4096, pos_hi=32767,
                                    seed=workload_seed(31)),
    # MTP verify: 2 tokens per request, 128 requests, 16K contexts
    "logits-mtp": LogitsWorkload("logits-mtp", requests=128, query_len=2, groups=4, heads=8,
                                 block=64, pages_per_req=256, pos_lo=8192, pos_hi=16382,
                                 seed=workload_seed(32)),
}


@dataclass
class LogitsInputs:
    w: LogitsWorkload
    query: torch.Tensor          # uint8 (e4m3 bytes) [rows, heads, 256]
    weights: torch.Tensor        # fp32 [rows, heads]
    summaries: torch.Tensor      # uint8 (e4m3 bytes) [pages, rpb, 256]
    scales: torch.Tensor         # fp32 [pages, rpb]
    block_table: torch.Tensor    # int32 [requests, pages_per_req]
    positions: torch.Tensor      # int32 [rows]


def make_logits_inputs(w: LogitsWorkload, device="cpu", seed: int | None = None,
                       summaries: torch.Tensor | None = None,
                       scales: torch.Tensor | None = None) -> LogitsInputs:
    """Block table = random permutation; token j of a request at first + j,
    first ~ U[pos_lo, pos_hi]; query and summaries = e4m3(N(0,1)); scales ~
    U[0.02, 0.1]; weights ~ N(0,1) / sqrt(heads)."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    table = rng.permutation(w.total_pages).astype(np.int32).reshape(w.requests, w.pages_per_req)
    first = rng.integers(w.pos_lo, w.pos_hi + 1, size=w.requests)
    req = np.repeat(np.arange(w.requests), w.query_len * w.groups)
    j = np.tile(np.repeat(np.arange(w.query_len), w.groups), w.requests)
    positions = (first[req] + j).astype(np.int32)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 2 + 1)
    if summaries is None:
        summaries = torch.empty((w.total_pages, w.rpb, 256), dtype=torch.uint8, device=device)
        for p0 in range(0, w.total_pages, 65536):
            p1 = min(w.total_pages, p0 + 65536)
            x = torch.randn((p1 - p0, w.rpb, 256), generator=gen, device=device)
            summaries[p0:p1] = x.to(torch.float8_e4m3fn).view(torch.uint8)
        scales = 0.02 + 0.08 * torch.rand((w.total_pages, w.rpb), generator=gen, device=device)
    gen.manual_seed(seed * 2)
    query = torch.randn((w.rows, w.heads, 256), generator=gen, device=device).to(
        torch.float8_e4m3fn).view(torch.uint8)
    weights = torch.randn((w.rows, w.heads), generator=gen, device=device) / math.sqrt(w.heads)
    return LogitsInputs(w=w, query=query, weights=weights, summaries=summaries, scales=scales,
                        block_table=torch.from_numpy(table).to(device),
                        positions=torch.from_numpy(positions).to(device))
