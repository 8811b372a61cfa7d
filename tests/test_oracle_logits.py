"""Pins of the decode indexer-logits oracle (CPU) to its reading
score[r, j] = sum_h w[r,h] * max(0, s_j * q[r,h] . k_j) over the row's
regions (-inf past them).  The formula itself is a reading of pages that do
not show the kernel (parity unpinned); these pins fix the oracle to it:
a vectorised torch route (its own e4m3 decode, einsum), closed forms,
masking, page renaming and linearity."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle
from oracle.hostprep import logits_host_problem
from sparse_paged_decode_02_amd import inputs as gen


def tiny(seed, **kw):
    base = dict(name="tiny-logits", requests=3, query_len=1, groups=2, heads=4, block=32,
                pages_per_req=5, pos_lo=0, pos_hi=150, seed=seed)
    base.update(kw)
    return gen.LogitsWorkload(**base)


def torch_route(inp):
    w = inp.w
    q = inp.query.view(torch.float8_e4m3fn).to(torch.float64)
    k = inp.summaries.view(torch.float8_e4m3fn).to(torch.float64)
    out = torch.full((w.rows, w.num_regions), -math.inf, dtype=torch.float64)
    for r in range(w.rows):
        req = r // (w.groups * w.query_len)
        n = min(int(inp.positions[r]) // w.region_tokens + 1, w.num_regions)
        if int(inp.positions[r]) < 0 or n <= 0:
            continue
        j = torch.arange(n)
        pages = inp.block_table[req].long()[j // w.rpb]
        kj = k[pages, j % w.rpb]                          # [n, 256]
        sj = inp.scales[pages, j % w.rpb].to(torch.float64)
        dots = torch.einsum("hd,jd->hj", q[r], kj)       # [heads, n]
        x = torch.clamp(dots * sj[None, :], min=0.0)
        out[r, :n] = (inp.weights[r].to(torch.float64)[:, None] * x).sum(0)
    return out.numpy()


@pytest.mark.parametrize("seed", range(12))
def test_matches_vectorised_torch_route(seed):
    rng = np.random.default_rng(seed)
    w = tiny(seed, query_len=int(rng.integers(1, 3)), groups=int(rng.integers(1, 4)),
             heads=int(rng.choice([1, 3, 8, 16])), block=int(rng.choice([16, 32, 64])),
             pos_lo=-3, pos_hi=5 * 64)
    inp = gen.make_logits_inputs(w)
    got = oracle.indexer_logits(logits_host_problem(inp))
    ref = torch_route(inp)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    m = np.isfinite(ref)
    np.testing.assert_allclose(got[m], ref[m], rtol=1e-12, atol=1e-12)


def test_closed_forms_and_relu():
    w = tiny(1, requests=1, groups=1, heads=2, block=16, pages_per_req=2, pos_lo=31, pos_hi=31)
    inp = gen.make_logits_inputs(w)
    inp.query.zero_()
    inp.summaries.zero_()
    one = 0x38   # e4m3 1.0
    inp.query[0, 0, 5] = one
    inp.query[0, 1, 7] = one
    table = inp.block_table.numpy()
    # region 1 (page table[0,0], slot 1): k[5] = 2.0 (0x40), k[7] = -2.0 (0xC0)
    inp.summaries[table[0, 0], 1, 5] = 0x40
    inp.summaries[table[0, 0], 1, 7] = 0xC0
    inp.scales.fill_(0.5)
    inp.weights[0] = torch.tensor([3.0, 5.0])
    got = oracle.indexer_logits(logits_host_problem(inp))[0]
    # head 0: relu(0.5 * 2) * 3 = 3; head 1: relu(0.5 * -2) * 5 = 0
    assert got[1] == 3.0
    assert (got[[0, 2, 3]] == 0.0).all()          # zero summaries score 0
    assert got.shape == (w.num_regions,)
    # position 31 with 8-token regions: regions 0..3 scored, the rest -inf
    assert np.isinf(got[4:]).all() and (got[4:] < 0).all()


def test_negative_positions_mask_everything():
    w = tiny(2, requests=2, groups=1, pos_lo=-5, pos_hi=-1)
    inp = gen.make_logits_inputs(w)
    got = oracle.indexer_logits(logits_host_problem(inp))
    assert np.isneginf(got).all()


def test_page_renaming_and_weight_linearity():
    w = tiny(3, pos_lo=40, pos_hi=150)
    inp = gen.make_logits_inputs(w)
    a = oracle.indexer_logits(logits_host_problem(inp))
    perm = torch.from_numpy(np.random.default_rng(0).permutation(w.total_pages))
    sm2 = torch.empty_like(inp.summaries)
    sm2[perm] = inp.summaries
    sc2 = torch.empty_like(inp.scales)
    sc2[perm] = inp.scales
    inp2 = gen.LogitsInputs(w=w, query=inp.query, weights=inp.weights, summaries=sm2,
                            scales=sc2, block_table=perm[inp.block_table.long()].to(torch.int32),
                            positions=inp.positions)
    np.testing.assert_array_equal(oracle.indexer_logits(logits_host_problem(inp2)), a)
    inp.weights.mul_(2.0)
    b = oracle.indexer_logits(logits_host_problem(inp))
    m = np.isfinite(a)
    np.testing.assert_array_equal(b[m], 2.0 * a[m])


def test_missing_page_is_refused():
    w = tiny(4, requests=1, pos_lo=100, pos_hi=100)
    inp = gen.make_logits_inputs(w)
    hp = logits_host_problem(inp)
    hp.block_table = hp.block_table.copy()
    hp.block_table[0, 0] = hp.summaries.shape[0]
    with pytest.raises(RuntimeError):
        oracle.indexer_logits(hp)
