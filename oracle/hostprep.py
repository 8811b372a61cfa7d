"""Host copies of decode inputs for the oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg).  It turns a
set of (possibly device-resident) input tensors into an oracle
``HostProblem``.  For caches too large to copy it ships only the pages that
the requested rows can reach.  The block table is then renumbered to index
the compact copy, and every entry no requested row needs is set to -1.  If
this bookkeeping ever missed a page, the oracle would refuse the row (page
id -1 is outside the copy) rather than compute a wrong value.
"""
from __future__ import annotations

import numpy as np
import torch

from .oracle import HostProblem, SwaHostProblem

_WHOLE_CACHE_BYTES = 256 << 20


def _bits16(t: torch.Tensor) -> np.ndarray:
    return np.array(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16),
                    copy=True)


def _needed_columns(regions, positions, active, rows, groups, query_len, block, rt):
    """(request, block-table column) pairs the given rows can touch."""
    need = set()
    per_req = groups * query_len
    for r in rows:
        if not active[r]:
            continue
        req = r // per_req
        pos = int(positions[r])
        for rid in regions[r]:
            rid = int(rid)
            if rid < 0:
                continue
            t0 = rid * rt
            if t0 > pos:
                continue
            t1 = min(t0 + rt - 1, pos)
            for col in range(t0 // block, t1 // block + 1):
                need.add((req, col))
    return need


def host_problem(query, cache, regions, block_table, positions, active, *, scale,
                 query_len=1, region_tokens=0, clear_inactive=True, k_scale=None,
                 v_scale=None, gate=None, rows=None) -> HostProblem:
    """Build the oracle's host problem.  ``rows``: the rows that will be
    evaluated (default all); with a large cache only their pages are copied.
    ``k_scale``/``v_scale`` may be floats or 1-element tensors."""
    # private copies: a CPU tensor's .numpy() shares its memory
    reg = np.array(regions.detach().cpu().numpy(), dtype=np.int32, copy=True)
    pos = np.array(positions.detach().cpu().numpy(), dtype=np.int32, copy=True)
    act = np.array(active.detach().cpu().numpy(), dtype=np.uint8, copy=True)
    table = np.array(block_table.detach().cpu().numpy(), dtype=np.int32, copy=True)
    groups, block = cache.shape[1], cache.shape[2]
    rt = region_tokens or block
    fp8 = cache.dtype in (torch.uint8, torch.float8_e4m3fn)
    cache_bytes = cache.numel() * cache.element_size()
    row_list = range(reg.shape[0]) if rows is None else [int(r) for r in rows]

    if cache_bytes <= _WHOLE_CACHE_BYTES:
        c = cache.detach().cpu().contiguous()
        host_cache = np.array(c.view(torch.uint8).numpy(), copy=True) if fp8 else _bits16(c)
        host_table = np.ascontiguousarray(table)
    else:
        need = _needed_columns(reg, pos, act, row_list, groups, query_len, block, rt)
        pages = sorted({int(table[q, c]) for q, c in need})
        remap = {p: i for i, p in enumerate(pages)}
        idx = torch.tensor(pages if pages else [0], dtype=torch.long, device=cache.device)
        sub = cache.index_select(0, idx).detach().cpu().contiguous()
        host_cache = sub.view(torch.uint8).numpy() if fp8 else _bits16(sub)
        if not pages:
            host_cache = host_cache[:0]
        host_table = np.full(table.shape, -1, dtype=np.int32)
        for q, c in need:
            host_table[q, c] = remap[int(table[q, c])]

    def _f(s):
        if s is None:
            return 1.0
        return float(s.detach().cpu().reshape(-1)[0]) if torch.is_tensor(s) else float(s)

    return HostProblem(
        query=_bits16(query),
        cache=host_cache,
        regions=np.ascontiguousarray(reg),
        block_table=host_table,
        positions=np.ascontiguousarray(pos),
        active=np.ascontiguousarray(act),
        scale=float(scale),
        query_len=int(query_len),
        region_tokens=int(region_tokens),
        clear_inactive=bool(clear_inactive),
        k_scale=_f(k_scale),
        v_scale=_f(v_scale),
        gate=None if gate is None else _bits16(gate),
    )


def host_problem_from_inputs(inp, rows=None, clear_inactive=True) -> HostProblem:
    """``host_problem`` for an ``Inputs`` bundle of the workload generator."""
    return host_problem(inp.query, inp.cache, inp.regions, inp.block_table, inp.positions,
                        inp.active, scale=inp.scale, query_len=inp.w.query_len,
                        region_tokens=inp.w.region_tokens, clear_inactive=clear_inactive,
                        k_scale=inp.k_scale, v_scale=inp.v_scale, gate=inp.gate, rows=rows)


def swa_host_problem(query, cache, block_table, seq_lens, *, scale, window, query_len=1,
                     gate=None, rows=None) -> SwaHostProblem:
    """The oracle's sliding-window problem.  ``query`` is [tokens, G*heads,
    192] as the attention layer holds it; the host copy is its row view
    [tokens*G, heads, 192].  With a large cache only the window pages of the
    ``rows`` to be evaluated are copied (block table renumbered, the rest -1)."""
    groups, block = cache.shape[1], cache.shape[2]
    tokens = query.shape[0]
    heads = query.shape[1] // groups
    table = np.array(block_table.detach().cpu().numpy(), dtype=np.int32, copy=True)
    lens = np.array(seq_lens.detach().cpu().numpy(), dtype=np.int32, copy=True)
    q = _bits16(query).reshape(tokens * groups, heads, query.shape[2])
    row_list = range(tokens * groups) if rows is None else [int(r) for r in rows]
    if cache.numel() * cache.element_size() <= _WHOLE_CACHE_BYTES:
        host_cache = _bits16(cache)
        host_table = np.ascontiguousarray(table)
    else:
        need = set()
        for r in row_list:
            t = r // groups
            req, j = t // query_len, t % query_len
            pos = int(lens[req]) - query_len + j
            if pos < 0:
                continue
            first = max(0, pos - window + 1)
            for col in range(first // block, pos // block + 1):
                need.add((req, col))
        pages = sorted({int(table[q_, c]) for q_, c in need})
        remap = {p: i for i, p in enumerate(pages)}
        idx = torch.tensor(pages if pages else [0], dtype=torch.long, device=cache.device)
        host_cache = _bits16(cache.index_select(0, idx))
        if not pages:
            host_cache = host_cache[:0]
        host_table = np.full(table.shape, -1, dtype=np.int32)
        for q_, c in need:
            host_table[q_, c] = remap[int(table[q_, c])]
    return SwaHostProblem(query=q, cache=host_cache, block_table=host_table,
                          seq_lens=np.ascontiguousarray(lens), scale=float(scale),
                          window=int(window), query_len=int(query_len),
                          gate=None if gate is None else _bits16(gate))


def logits_host_problem(inp, rows=None):
    """The oracle's indexer-logits problem for a LogitsInputs bundle.  With a
    large summary cache only the pages the ``rows`` can reach are copied
    (block table renumbered, other entries -1)."""
    from .oracle import LogitsHostProblem
    w = inp.w
    table = np.array(inp.block_table.detach().cpu().numpy(), dtype=np.int32, copy=True)
    pos = np.array(inp.positions.detach().cpu().numpy(), dtype=np.int32, copy=True)
    row_list = range(w.rows) if rows is None else [int(r) for r in rows]
    sm, sc = inp.summaries, inp.scales
    if sm.numel() <= _WHOLE_CACHE_BYTES:
        host_sm = np.array(sm.detach().cpu().numpy(), copy=True)
        host_sc = np.array(sc.detach().cpu().numpy(), dtype=np.float32, copy=True)
        host_table = np.ascontiguousarray(table)
    else:
        need = set()
        per_req = w.groups * w.query_len
        for r in row_list:
            req = r // per_req
            if pos[r] < 0:
                continue
            last = min(int(pos[r]) // w.region_tokens, w.num_regions - 1)
            for col in range(last // w.rpb + 1):
                need.add((req, col))
        pages = sorted({int(table[q, c]) for q, c in need})
        remap = {p: i for i, p in enumerate(pages)}
        idx = torch.tensor(pages if pages else [0], dtype=torch.long, device=sm.device)
        host_sm = np.array(sm.index_select(0, idx).cpu().numpy(), copy=True)
        host_sc = np.array(sc.index_select(0, idx).cpu().numpy(), dtype=np.float32, copy=True)
        if not pages:
            host_sm, host_sc = host_sm[:0], host_sc[:0]
        host_table = np.full(table.shape, -1, dtype=np.int32)
        for q, c in need:
            host_table[q, c] = remap[int(table[q, c])]
    return LogitsHostProblem(
        query=np.array(inp.query.detach().cpu().numpy(), copy=True),
        weights=np.array(inp.weights.detach().cpu().numpy(), dtype=np.float32, copy=True),
        summaries=host_sm, scales=host_sc, block_table=host_table, positions=pos,
        groups=w.groups, num_regions=w.num_regions, query_len=w.query_len,
        region_tokens=w.region_tokens)
