"""Pins of the sliding-window oracle (CPU): a band-masked dense SDPA by
another route, the full-context limit against the (separately pinned) sparse
oracle, closed forms for window 1 and for one-hot values, and the token
positions of multi-token requests."""
import numpy as np
import pytest
import torch

from oracle import oracle
from oracle.hostprep import host_problem, swa_host_problem
from sparse_paged_decode_02_amd import inputs as gen
from _util import DIM, swa_dense_reference, swa_gate_values


def tiny_swa(seed, **kw):
    base = dict(name="tiny-swa", requests=3, query_len=1, groups=2, heads=4, block=16,
                pages_per_req=6, window=20, seq_lo=1, seq_hi=96, gated=True, splits=1,
                seed=seed)
    base.update(kw)
    return gen.SwaWorkload(**base)


def _hp(inp, **kw):
    return swa_host_problem(inp.query, inp.cache, inp.block_table, inp.seq_lens,
                            scale=inp.scale, window=inp.w.window, query_len=inp.w.query_len,
                            gate=inp.gate, **kw)


def _random_swa(seed):
    rng = np.random.default_rng(seed)
    block = int(rng.choice([4, 8, 16, 32]))
    pages = int(rng.integers(2, 6))
    qlen = int(rng.choice([1, 2, 3, 4]))
    w = tiny_swa(seed, requests=int(rng.integers(1, 4)), query_len=qlen,
                 groups=int(rng.choice([1, 2, 3])), heads=int(rng.choice([1, 3, 8, 16])),
                 block=block, pages_per_req=pages,
                 window=int(rng.choice([1, 2, 7, block, block + 1, 3 * block, 1000])),
                 seq_lo=qlen, seq_hi=pages * block, gated=bool(rng.random() < 0.5))
    return w


@pytest.mark.parametrize("seed", range(40))
def test_swa_oracle_matches_band_sdpa(seed):
    w = _random_swa(seed)
    inp = gen.make_swa_inputs(w)
    hp = _hp(inp)
    got = oracle.swa_decode(hp)
    ref = swa_dense_reference(hp, swa_gate_values(hp))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)


def test_full_window_equals_sparse_oracle_over_all_pages():
    # window >= context: every causally visible token, i.e. the sparse
    # definition with every page of the request selected
    w = tiny_swa(3, query_len=2, window=10_000, seq_lo=2, seq_hi=96)
    inp = gen.make_swa_inputs(w)
    hp = _hp(inp)
    got = oracle.swa_decode(hp)
    G, ppr = w.groups, w.pages_per_req
    rows = w.rows
    tok = np.arange(rows) // G
    req, j = tok // w.query_len, tok % w.query_len
    pos = inp.seq_lens.numpy()[req] - w.query_len + j
    regions = torch.from_numpy(np.tile(np.arange(ppr, dtype=np.int32), (rows, 1)))
    q_rows = inp.query.reshape(rows, w.heads, DIM)
    sp = host_problem(q_rows, inp.cache, regions, inp.block_table,
                      torch.from_numpy(pos.astype(np.int32)), torch.ones(rows, dtype=torch.bool),
                      scale=inp.scale, query_len=w.query_len, gate=inp.gate)
    ref = oracle.decode(sp)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_window_one_returns_the_current_value():
    w = tiny_swa(5, query_len=3, window=1, seq_lo=3, seq_hi=96, gated=False)
    inp = gen.make_swa_inputs(w)
    hp = _hp(inp)
    got = oracle.swa_decode(hp)
    c = torch.from_numpy(hp.cache.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    for r in range(w.rows):
        t, g = r // w.groups, r % w.groups
        req, j = t // w.query_len, t % w.query_len
        pos = int(hp.seq_lens[req]) - w.query_len + j
        v = c[hp.block_table[req, pos // w.block], g, pos % w.block, DIM:].numpy()
        assert np.array_equal(got[r], np.broadcast_to(v, got[r].shape))


def test_one_hot_values_reveal_the_window_exactly():
    # q = 0 gives uniform weights; V[t] = e_(t mod 192) makes out[d] the
    # fraction of window tokens congruent to d: the window's exact extent.
    w = tiny_swa(7, requests=4, query_len=4, groups=1, heads=2, block=8, pages_per_req=32,
                 window=37, seq_lo=4, seq_hi=256, gated=False)
    inp = gen.make_swa_inputs(w, seq_lens=[4, 37, 40, 256])
    inp.query.zero_()
    table = inp.block_table.numpy()
    inp.cache.zero_()
    for req in range(w.requests):
        for t in range(w.pages_per_req * w.block):
            inp.cache[table[req, t // w.block], 0, t % w.block, DIM + t % DIM] = 1.0
    hp = _hp(inp)
    got = oracle.swa_decode(hp)
    for r in range(w.rows):
        req, j = r // w.query_len, r % w.query_len
        pos = int(hp.seq_lens[req]) - w.query_len + j
        toks = np.arange(max(0, pos - w.window + 1), pos + 1)
        want = np.bincount(toks % DIM, minlength=DIM) / len(toks)
        for h in range(w.heads):
            np.testing.assert_allclose(got[r, h], want, rtol=0, atol=1e-15)


def test_gate_scales_each_head():
    w = tiny_swa(9, gated=True)
    inp = gen.make_swa_inputs(w)
    hp = _hp(inp)
    gated = oracle.swa_decode(hp)
    hp.gate = None
    plain = oracle.swa_decode(hp)
    hp.gate = _hp(inp).gate
    gv = swa_gate_values(hp)
    np.testing.assert_array_equal(gated, plain * gv[:, :, None])


def test_page_renaming_is_invisible():
    w = tiny_swa(13, query_len=2, seq_lo=2)
    inp = gen.make_swa_inputs(w)
    a = oracle.swa_decode(_hp(inp))
    perm = torch.from_numpy(np.random.default_rng(1).permutation(w.total_pages))
    cache2 = torch.empty_like(inp.cache)
    cache2[perm] = inp.cache
    inp.block_table = perm[inp.block_table.long()].to(torch.int32)
    inp.cache = cache2
    b = oracle.swa_decode(_hp(inp))
    np.testing.assert_array_equal(a, b)


def test_missing_page_is_refused():
    w = tiny_swa(17, seq_lo=40, seq_hi=40, window=30)
    inp = gen.make_swa_inputs(w)
    hp = _hp(inp)
    hp.block_table = hp.block_table.copy()
    hp.block_table[0, 1] = hp.cache.shape[0]   # the window of request 0 uses column 1
    with pytest.raises(RuntimeError):
        oracle.swa_decode(hp, rows=[0])
