"""GPU parity of the gated sliding-window decode (sda_swa_decode) against the
fp64 oracle (MI355X).

Floating point: max |gpu - oracle| <= 1.5e-2 and mean <= 1e-3 on bf16 outputs.
The window's extent (which positions each token sees) is checked exactly
through one-hot values, and rows without a visible token through exact zeros.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from oracle.hostprep import swa_host_problem
from sparse_paged_decode_02_amd import binding as B
from sparse_paged_decode_02_amd import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_ABS = 1.5e-2
MEAN_ABS = 1e-3
ORACLE_THREADS = 16
DIM = 192


def _say(msg):
    sys.stderr.write("[swa] %s\n" % msg)
    sys.stderr.flush()


def case(seed, **kw):
    base = dict(name="swa-case", requests=3, query_len=1, groups=2, heads=16, block=64,
                pages_per_req=12, window=300, seq_lo=1, seq_hi=768, gated=True, splits=None,
                seed=seed)
    base.update(kw)
    return gen.SwaWorkload(**base)


def run(inp, splits=None, query=None, out=None, gate="inp", label="", pack=0):
    w = inp.w
    if splits is None:
        splits = inp.splits if inp.splits is not None else B.sda_swa_plan(
            w.tokens, w.groups, w.heads, w.query_len, w.window)[1]
    q = inp.query if query is None else query
    if out is None:
        out = torch.empty_like(inp.query)
    g = inp.gate if gate == "inp" else gate
    _say("sda_swa_decode %s tokens=%d G=%d heads=%d block=%d window=%d qlen=%d splits=%d "
         "pack=%d gate=%s" % (label or w.name, w.tokens, w.groups, w.heads, w.block, w.window,
                              w.query_len, splits, pack, g is not None))
    B.sda_swa_decode(q, inp.cache, inp.block_table, inp.seq_lens, out, scale=inp.scale,
                     window=w.window, query_len=w.query_len, splits=splits, pack=pack, gate=g)
    torch.cuda.synchronize()
    return out


def oracle_out(inp, rows=None, gate="inp"):
    g = inp.gate if gate == "inp" else gate
    hp = swa_host_problem(inp.query, inp.cache, inp.block_table, inp.seq_lens, scale=inp.scale,
                          window=inp.w.window, query_len=inp.w.query_len, gate=g, rows=rows)
    return oracle.swa_decode(hp, rows=rows, threads=ORACLE_THREADS)


def as_rows(out, w):
    """[tokens, G*heads, 192] -> [rows, heads, 192] float64 numpy."""
    return out.detach().float().cpu().numpy().astype(np.float64).reshape(w.rows, w.heads, DIM)


def check_close(gpu, ref, w, rows=None, what=""):
    g = as_rows(gpu, w)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert not np.isnan(ref).any(), "oracle left rows unset"
    err = np.abs(g - ref)
    _say("%s max_abs=%.3e mean_abs=%.3e" % (what, err.max(), err.mean()))
    assert err.max() <= MAX_ABS, (what, err.max())
    assert err.mean() <= MEAN_ABS, (what, err.mean())


# ---------------------------------------------------------------------------
def _random_case(seed):
    rng = np.random.default_rng(seed)
    block = int(rng.choice([16, 32, 64]))
    pages = int(rng.integers(3, 12))
    qlen = int(rng.choice([1, 2, 3, 4]))
    ctx = pages * block
    window = int(rng.choice([1, 5, 16, 17, 63, 100, 257, ctx + 50]))
    return case(seed, requests=int(rng.integers(1, 5)), query_len=qlen,
                groups=int(rng.choice([1, 2, 4])), heads=int(rng.choice([1, 4, 8, 13, 16])),
                block=block, pages_per_req=pages, window=window, seq_lo=qlen, seq_hi=ctx,
                gated=bool(rng.random() < 0.7))


@pytest.mark.parametrize("seed", range(24))
def test_random_cases_match_oracle(seed):
    w = _random_case(seed)
    inp = gen.make_swa_inputs(w, device=DEV)
    splits = [1, 2, 3, 5][seed % 4]
    pack = int(np.random.default_rng(seed + 1000).integers(0, min(w.query_len,
                                                                  16 // w.heads) + 1))
    out = run(inp, splits=splits, label="random%d" % seed, pack=pack)
    check_close(out, oracle_out(inp), w, what="random%d" % seed)


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 7, 16, 40])
def test_split_sweep(splits):
    w = case(101, requests=2, query_len=2, window=700, seq_lo=600, seq_hi=768)
    inp = gen.make_swa_inputs(w, device=DEV)
    out = run(inp, splits=splits)
    check_close(out, oracle_out(inp), w, what="splits%d" % splits)


@pytest.mark.parametrize("heads,pack", [(4, 1), (4, 2), (4, 3), (4, 4), (3, 0), (8, 2),
                                        (16, 1)])
@pytest.mark.parametrize("splits", [1, 3])
def test_token_packing(heads, pack, splits):
    # the query tokens of a request share one workgroup, each with its own
    # window mask; windows straddle page and chunk edges
    w = case(31 + heads, requests=3, query_len=4, groups=2, heads=heads, block=32,
             pages_per_req=20, window=70, gated=True)
    inp = gen.make_swa_inputs(w, device=DEV, seq_lens=[4, 75, 640])
    out = run(inp, splits=splits, pack=pack, label="pack%d" % pack)
    check_close(out, oracle_out(inp), w, what="heads%d pack%d splits%d" % (heads, pack, splits))


@pytest.mark.parametrize("splits", [1, 2])
def test_packed_column_empty_in_one_wave(splits):
    # seq_len 33, query_len 2, window 16: token 0 sees 16..31 and token 1
    # sees 17..32.  The union's second chunk (32..47) holds a visible token
    # for token 1 only, so the wave computing it has token 0's columns still
    # empty while token 1's columns raise the running max.
    w = case(41, requests=2, query_len=2, groups=2, heads=8, block=16, pages_per_req=4,
             window=16, gated=True)
    inp = gen.make_swa_inputs(w, device=DEV, seq_lens=[33, 49])
    out = run(inp, splits=splits, pack=2, label="empty column")
    assert torch.isfinite(out.float()).all()
    check_close(out, oracle_out(inp), w, what="empty column splits%d" % splits)


@pytest.mark.parametrize("pack", [1, 4])
@pytest.mark.parametrize("splits", [1, 3])
def test_window_extent_exact(splits, pack):
    # q = 0: uniform weights; V[t] = 1 at dim t % 192, so the output's support
    # is exactly the set of window positions mod 192 (window <= 192).
    w = case(7, requests=4, query_len=4, groups=2, heads=3, block=16, pages_per_req=24,
             window=37, gated=False)
    assert pack <= 16 // w.heads
    inp = gen.make_swa_inputs(w, device=DEV, seq_lens=[4, 37, 40, 384])
    inp.query.zero_()
    cache = torch.zeros_like(inp.cache)
    table = inp.block_table.cpu().numpy()
    for req in range(w.requests):
        for t in range(w.pages_per_req * w.block):
            cache[table[req, t // w.block], :, t % w.block, DIM + t % DIM] = 1.0
    inp.cache = cache
    out = as_rows(run(inp, splits=splits, pack=pack), w)
    lens = [4, 37, 40, 384]
    for r in range(w.rows):
        tok = r // w.groups
        req, j = tok // w.query_len, tok % w.query_len
        pos = lens[req] - w.query_len + j
        toks = np.arange(max(0, pos - w.window + 1), pos + 1)
        support = np.zeros(DIM, bool)
        support[toks % DIM] = True
        for h in range(w.heads):
            assert np.array_equal(out[r, h] != 0, support), (r, h)
            np.testing.assert_allclose(out[r, h][support], 1.0 / len(toks), rtol=8e-3)


def test_tokens_before_the_first_position_are_zero():
    # seq_len < query_len: the leading tokens have negative positions and no
    # visible token; their outputs are exact zeros.
    w = case(9, requests=3, query_len=4, groups=2, heads=4, block=16, pages_per_req=4,
             window=20)
    inp = gen.make_swa_inputs(w, device=DEV, seq_lens=[1, 2, 50])
    out = run(inp, splits=2, pack=3)
    ref = oracle_out(inp)
    check_close(out, ref, w, what="short requests")
    o = as_rows(out, w)
    for r in range(w.rows):
        tok = r // w.groups
        req, j = tok // w.query_len, tok % w.query_len
        if [1, 2, 50][req] - w.query_len + j < 0:
            assert (o[r] == 0).all()


def test_strided_query_and_output_views():
    # query as a slice of a wider projection output (token stride > heads*192),
    # output as a slice of a wider buffer
    w = case(13, requests=3, query_len=2, groups=2, heads=8, window=200)
    inp = gen.make_swa_inputs(w, device=DEV)
    H = w.groups * w.heads
    wide = torch.randn((w.tokens, H + 5, DIM), device=DEV).to(torch.bfloat16)
    wide[:, 3:3 + H] = inp.query
    q = wide[:, 3:3 + H]
    obuf = torch.full((w.tokens, H + 2, DIM), 7.0, device=DEV, dtype=torch.bfloat16)
    o = obuf[:, 1:1 + H]
    gwide = torch.zeros((w.tokens, H + 4), device=DEV, dtype=torch.bfloat16)
    gwide[:, 2:2 + H] = inp.gate
    run(inp, query=q, out=o, gate=gwide[:, 2:2 + H], splits=2)
    ref_out = run(inp, splits=2)
    assert torch.equal(o, ref_out)
    assert (obuf[:, 0] == 7.0).all() and (obuf[:, H + 1] == 7.0).all()


def test_full_window_matches_sparse_decode():
    # window >= context: the same rows through sda_decode with every page of
    # the request selected give the same result (same kernel arithmetic
    # order is not required, so compare to the bar, not bitwise)
    w = case(17, requests=2, query_len=2, groups=2, heads=16, pages_per_req=6,
             window=10_000, seq_lo=2, seq_hi=384, gated=True)
    inp = gen.make_swa_inputs(w, device=DEV)
    out = run(inp, splits=1)
    rows = w.rows
    tok = torch.arange(rows) // w.groups
    req, j = tok // w.query_len, tok % w.query_len
    pos = (inp.seq_lens.cpu().long()[req] - w.query_len + j).to(torch.int32)
    regions = torch.arange(w.pages_per_req, dtype=torch.int32).repeat(rows, 1)
    sp_out = torch.empty((rows, w.heads, DIM), device=DEV, dtype=torch.bfloat16)
    B.sda_decode(inp.query.reshape(rows, w.heads, DIM), inp.cache, regions.to(DEV),
                 inp.block_table, pos.to(DEV), torch.ones(rows, dtype=torch.bool, device=DEV),
                 sp_out, scale=inp.scale, query_len=w.query_len, splits=1, gate=inp.gate)
    torch.cuda.synchronize()
    d = (out.reshape(rows, w.heads, DIM).float() - sp_out.float()).abs()
    assert d.max().item() <= MAX_ABS and d.mean().item() <= MEAN_ABS


def test_empty_batch_is_noop():
    w = case(19, requests=1)
    inp = gen.make_swa_inputs(w, device=DEV)
    q = inp.query[:0]
    out = torch.empty_like(q)
    B.sda_swa_decode(q, inp.cache, inp.block_table, inp.seq_lens, out, scale=inp.scale,
                     window=w.window, query_len=1, splits=1, gate=None)
    torch.cuda.synchronize()


@pytest.mark.parametrize("qlen,heads,splits", [(1, 16, 1), (4, 4, 2), (2, 16, 1)])
def test_large_grid_variant(qlen, heads, splits):
    # >= 512 workgroups: the 2-wave kernel variant
    w = case(61, requests=160, query_len=qlen, groups=4, heads=heads, block=16,
             pages_per_req=8, window=50, seq_lo=qlen, seq_hi=128)
    inp = gen.make_swa_inputs(w, device=DEV)
    out = run(inp, splits=splits, label="large grid")
    check_close(out, oracle_out(inp), w, what="large grid q%d h%d s%d" % (qlen, heads, splits))


# --- full-size workloads: sampled rows + properties ---------------------------
@pytest.mark.parametrize("name", ["swa-gated", "swa-mtp"])
def test_full_size_sampled(name):
    w = gen.SWA_WORKLOADS[name]
    _say("drawing full workload %s" % name)
    inp = gen.make_swa_inputs(w, device=DEV)
    out = run(inp, label="full " + name)
    rng = np.random.default_rng(len(name))
    rows = sorted(set(rng.choice(w.rows, size=min(24, w.rows), replace=False).tolist()
                      + [0, w.rows - 1]))
    check_close(out, oracle_out(inp, rows=rows), w, rows=rows, what=name + " sampled")
    o = out.float()
    assert torch.isfinite(o).all()
    assert o.abs().max().item() <= 8.0
    del inp, out
    torch.cuda.empty_cache()
