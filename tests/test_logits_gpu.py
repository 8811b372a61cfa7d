"""GPU parity of the decode indexer logits (sda_indexer_logits) against the
fp64 oracle (MI355X), and of the whole upstream chain logits -> selection ->
decode.

Tolerance, from the arithmetic: the e4m3 products are exact, the 256-term dot
is summed in fp32, then scaled, weighted and summed over <= 16 heads, so
|gpu - oracle| <= ~276 * 2^-24 * B with B = sum_h |w_h| |s_j| sum_d |q_hd k_jd|;
the test allows 2^-15 * B.  Masked columns (-inf) and the current / length
outputs are compared exactly."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from oracle.hostprep import host_problem, logits_host_problem
from sparse_paged_decode_02_amd import binding as B
from sparse_paged_decode_02_amd import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    sys.stderr.write("[logits] %s\n" % msg)
    sys.stderr.flush()


def run(inp, scores=None, query=None, label="", table=None, table_cols=None):
    w = inp.w
    rows = w.rows
    cur = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    lens = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    _say("sda_indexer_logits %s rows=%d heads=%d G=%d qlen=%d rpb=%d S=%d" % (
        label or w.name, rows, w.heads, w.groups, w.query_len, w.rpb, w.num_regions))
    out = B.sda_indexer_logits(inp.query if query is None else query, inp.weights, inp.summaries,
                               inp.scales, inp.block_table if table is None else table,
                               inp.positions, groups=w.groups,
                               num_regions=w.num_regions, query_len=w.query_len,
                               region_tokens=w.region_tokens, scores=scores, current=cur,
                               topk_lengths=lens, table_cols=table_cols)
    torch.cuda.synchronize()
    return out, cur, lens


def abs_bound(inp, rows):
    """B[r, j] of the tolerance (float64), from torch's own e4m3 decode."""
    w = inp.w
    q = inp.query.cpu().view(torch.float8_e4m3fn).to(torch.float64).abs()
    k = inp.summaries.cpu().view(torch.float8_e4m3fn).to(torch.float64).abs()
    bt = inp.block_table.cpu().long()
    out = np.zeros((len(rows), w.num_regions))
    j = torch.arange(w.num_regions)
    for i, r in enumerate(rows):
        req = r // (w.groups * w.query_len)
        col = (j // w.rpb).clamp(max=bt.shape[1] - 1)
        pages = bt[req][col]
        kj = k[pages, j % w.rpb]
        sj = inp.scales.cpu()[pages, j % w.rpb].to(torch.float64).abs()
        dots = torch.einsum("hd,jd->hj", q[r], kj) * sj[None, :]
        out[i] = (inp.weights.cpu()[r].to(torch.float64).abs()[:, None] * dots).sum(0).numpy()
    return out


def check(inp, got, cur, lens, rows=None, what=""):
    w = inp.w
    rows = list(range(w.rows)) if rows is None else rows
    ref = oracle.indexer_logits(logits_host_problem(inp, rows=rows), rows=rows, threads=16)[rows]
    g = got.cpu().numpy().astype(np.float64)[rows]
    inf_ref, inf_got = np.isneginf(ref), np.isneginf(g)
    assert np.array_equal(inf_ref, inf_got), what
    m = ~inf_ref
    bound = abs_bound(inp, rows)
    err = np.where(m, np.abs(np.where(m, g, 0.0) - np.where(m, ref, 0.0)), 0.0)
    _say("%s max_err=%.3e max_err/B=%.3e" % (what, err[m].max() if m.any() else 0.0,
                                                (err[m] / np.maximum(bound[m], 1e-30)).max()
                                                if m.any() else 0.0))
    assert (err[m] <= 2.0 ** -15 * bound[m] + 1e-30).all(), what
    pos = inp.positions.cpu().numpy()[rows].astype(np.int64)
    c = np.where(pos < 0, -1, pos // w.region_tokens)
    assert np.array_equal(cur.cpu().numpy()[rows], c)
    assert np.array_equal(lens.cpu().numpy()[rows], np.minimum(c + 1, w.num_regions))


def case(seed, **kw):
    base = dict(name="logits-case", requests=3, query_len=1, groups=2, heads=8, block=64,
                pages_per_req=12, pos_lo=0, pos_hi=12 * 64 - 1, seed=seed)
    base.update(kw)
    return gen.LogitsWorkload(**base)


@pytest.mark.parametrize("heads,groups,qlen", [(1, 1, 1), (2, 3, 1), (4, 4, 1), (8, 4, 1),
                                               (8, 4, 2), (16, 2, 2), (16, 4, 1), (4, 2, 4)])
@pytest.mark.parametrize("block", [16, 64])
def test_shapes(heads, groups, qlen, block):
    w = case(heads * 10 + groups + block, heads=heads, groups=groups, query_len=qlen, block=block,
             pages_per_req=40 if block == 16 else 12, pos_lo=-2,
             pos_hi=(40 if block == 16 else 12) * block - qlen)
    inp = gen.make_logits_inputs(w, device=DEV)
    got, cur, lens = run(inp)
    check(inp, got, cur, lens, what="h%d g%d q%d b%d" % (heads, groups, qlen, block))


def test_ragged_columns_and_strided_views():
    # S not a multiple of 16 or 256 through a wider score buffer; padded query rows
    w = case(5, requests=4, groups=2, heads=8, block=32, pages_per_req=33, pos_lo=500,
             pos_hi=33 * 32 - 1)
    inp = gen.make_logits_inputs(w, device=DEV)
    S = w.num_regions   # 132
    buf = torch.full((w.rows, S + 12), 7.0, device=DEV)
    qbig = torch.zeros((w.rows, 10, 256 + 32), dtype=torch.uint8, device=DEV)
    qbig[:, :w.heads, 16:272] = inp.query
    got, cur, lens = run(inp, scores=buf[:, :S], query=qbig[:, :w.heads, 16:272])
    check(inp, got, cur, lens, what="strided")
    assert (buf[:, S:] == 7.0).all()


def test_scores_rows_of_any_stride():
    # Score rows are stored 4 bytes at a time: S = 594 (not a multiple of 4)
    # in a contiguous buffer, and the same in a view one float into a wider
    # buffer (rows 4-byte but not 16-byte aligned).
    w = case(17, requests=2, groups=2, heads=2, query_len=2, block=16, pages_per_req=297,
             pos_lo=459, pos_hi=297 * 16 - 2)
    inp = gen.make_logits_inputs(w, device=DEV)
    S = w.num_regions
    assert S % 4 == 2
    got, cur, lens = run(inp, scores=torch.empty((w.rows, S), device=DEV))
    check(inp, got, cur, lens, what="stride S")
    buf = torch.full((w.rows, S + 3), 7.0, device=DEV)
    got, cur, lens = run(inp, scores=buf[:, 1:S + 1])
    check(inp, got, cur, lens, what="stride S + 3, offset 1")
    assert (buf[:, 0] == 7.0).all() and (buf[:, S + 1:] == 7.0).all()


@pytest.mark.parametrize("requests,qlen", [(256, 1), (257, 1), (300, 2)])
def test_many_requests(requests, qlen):
    # Grids of 256 to 300 requests of 80 regions (a partial 256-region chunk
    # each), lengths from 0 to the whole row, every row.
    w = case(900 + requests, requests=requests, query_len=qlen, groups=2, heads=4, block=16,
             pages_per_req=40, pos_lo=-3, pos_hi=40 * 16 - qlen)
    inp = gen.make_logits_inputs(w, device=DEV)
    got, cur, lens = run(inp, label="requests=%d" % requests)
    check(inp, got, cur, lens, what="requests=%d qlen=%d" % (requests, qlen))


def test_no_live_region():
    # Every position negative: no live tile anywhere, every column -inf.
    w = case(31, requests=6, groups=2, heads=8, pos_lo=-40, pos_hi=-1)
    inp = gen.make_logits_inputs(w, device=DEV)
    got, cur, lens = run(inp, label="no live region")
    assert torch.isneginf(got).all()
    check(inp, got, cur, lens, what="no live region")


def test_long_row():
    # One request of 327680 regions (1280 chunks of 256), every one live:
    # the row against the oracle in full.
    w = case(77, requests=1, groups=1, heads=2, block=64, pages_per_req=40960,
             pos_lo=40960 * 64 - 1, pos_hi=40960 * 64 - 1)
    inp = gen.make_logits_inputs(w, device=DEV)
    got, cur, lens = run(inp, label="long row")
    check(inp, got, cur, lens, what="long row")


@pytest.mark.parametrize("name", ["logits-decode", "logits-mtp"])
def test_full_size_sampled(name):
    w = gen.LOGITS_WORKLOADS[name]
    inp = gen.make_logits_inputs(w, device=DEV)
    got, cur, lens = run(inp, label=name)
    rng = np.random.default_rng(len(name))
    rows = sorted(set(rng.choice(w.rows, size=12, replace=False).tolist() + [0, w.rows - 1]))
    check(inp, got, cur, lens, rows=rows, what=name + " sampled")
    # properties on every row: finite up to the row's length, -inf after
    g = got.cpu().numpy()
    L = lens.cpu().numpy()
    col = np.arange(w.num_regions)[None, :]
    assert np.isfinite(g[col < L[:, None]]).all()
    assert np.isneginf(g[col >= L[:, None]]).all()


def test_chain_logits_select_decode():
    # indexer logits -> region selection -> sparse decode at 8-token regions,
    # each stage compared with the oracle on the previous GPU stage's output
    # (the selection decides on the GPU's fp32 scores on both sides)
    dw = gen.Workload("chain", requests=4, query_len=1, groups=4, heads=16, block=64,
                      pages_per_req=24, R=96, kv="bf16", pos_lo=800, pos_hi=24 * 64 - 1,
                      gated=True, splits=1, region_tokens=8, seed=91)
    dec = gen.make_inputs(dw, device=DEV)
    lw = gen.LogitsWorkload("chain-logits", requests=4, query_len=1, groups=4, heads=8, block=64,
                            pages_per_req=24, pos_lo=0, pos_hi=1, seed=92)
    li = gen.make_logits_inputs(lw, device=DEV)
    li.block_table = dec.block_table
    li.positions = dec.positions
    scores, cur, lens = run(li, label="chain")
    check(li, scores, cur, lens, what="chain logits")
    regions = B.sda_select_regions(scores, cur, dw.R, topk_lengths=lens)
    torch.cuda.synchronize()
    ref_regions = oracle.select_regions(scores.cpu().numpy(), cur.cpu().numpy(), dw.R,
                                        lens.cpu().numpy())
    assert np.array_equal(regions.cpu().numpy(), ref_regions)
    out = torch.empty_like(dec.query)
    B.sda_decode(dec.query, dec.cache, regions, dec.block_table, dec.positions, dec.active, out,
                 scale=dec.scale, splits=1, gate=dec.gate, region_tokens=8)
    torch.cuda.synchronize()
    hp = host_problem(dec.query, dec.cache, torch.from_numpy(ref_regions), dec.block_table,
                      dec.positions, dec.active, scale=dec.scale, region_tokens=8,
                      gate=dec.gate)
    ref = oracle.decode(hp, threads=16)
    err = np.abs(out.float().cpu().numpy() - ref)
    assert err.max() <= 1.5e-2 and err.mean() <= 1e-3


@pytest.mark.parametrize("heads,groups,qlen", [(8, 4, 1), (8, 4, 2), (16, 2, 1)])
def test_table_cols_given_or_not(heads, groups, qlen):
    # With the table's column count a workgroup requests its table entries
    # beside the positions; with 0 only after them.  The same entries are
    # used either way: the scores must agree bit for bit.
    w = case(60 + heads + groups + qlen, requests=5, heads=heads, groups=groups, query_len=qlen,
             block=64, pages_per_req=48, pos_lo=-1, pos_hi=48 * 64 - qlen)
    inp = gen.make_logits_inputs(w, device=DEV)
    early, cur_e, lens_e = run(inp, label="table cols given")
    late, cur_l, lens_l = run(inp, label="table cols 0", table_cols=0)
    assert torch.equal(early.view(torch.int32), late.view(torch.int32))
    assert torch.equal(cur_e, cur_l) and torch.equal(lens_e, lens_l)
    check(inp, early, cur_e, lens_e, what="table cols h%d g%d q%d" % (heads, groups, qlen))


def test_table_narrower_than_the_score_columns():
    # A table with only the columns the scored regions need (21 of the 40
    # pages that the 320 score columns span): entries past them are never
    # requested, early or late.
    w = case(71, requests=4, heads=8, groups=4, block=64, pages_per_req=40, pos_lo=600,
             pos_hi=21 * 64 - 1)
    inp = gen.make_logits_inputs(w, device=DEV)
    narrow = inp.block_table[:, :21].contiguous()
    for cols in (None, 0):
        got, cur, lens = run(inp, label="narrow table cols=%s" % cols, table=narrow,
                             table_cols=cols)
        check(inp, got, cur, lens, what="narrow table cols=%s" % cols)
