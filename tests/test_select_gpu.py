"""GPU parity of region selection (sda_select_regions) against the oracle
(MI355X).  Selection is index work: the output must equal the oracle's bit
for bit, ties included (equal scores go to the lower region id)."""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle
from sparse_paged_decode_02_amd import binding as B
from sparse_paged_decode_02_amd import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    sys.stderr.write("[select] %s\n" % msg)
    sys.stderr.flush()


def run_and_check(scores, current, topk, lengths=None, label=""):
    rows, S = scores.shape
    _say("sda_select_regions %s rows=%d S=%d topk=%d lengths=%s" % (
        label, rows, S, topk, lengths is not None))
    out = B.sda_select_regions(scores.to(DEV), current.to(DEV), topk,
                               topk_lengths=None if lengths is None else lengths.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.select_regions(scores.cpu().numpy(), current.cpu().numpy(), topk,
                                None if lengths is None else lengths.cpu().numpy())
    got = out.cpu().numpy()
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert len(bad) == 0, (label, bad[:5], got[bad[0]][:20] if len(bad) else None,
                           ref[bad[0]][:20] if len(bad) else None)
    return got


def _case(seed, rows, S, dist):
    g = torch.Generator().manual_seed(seed)
    if dist == "normal":
        s = torch.randn((rows, S), generator=g)
    elif dist == "ties":
        s = torch.randint(0, 5, (rows, S), generator=g).float()
    elif dist == "zeros":
        s = torch.zeros((rows, S))
        s[:, 1::2] = -0.0
    else:  # wide dynamic range, infinities
        s = torch.randn((rows, S), generator=g) * torch.exp2(torch.randint(-60, 60, (rows, S),
                                                                          generator=g).float())
        s[:, ::7] = -float("inf")
        s[:, 3::11] = float("inf")
    return s.float()


@pytest.mark.parametrize("S", [1, 7, 256, 257, 1000, 2048, 4096, 8191, 16384, 32768])
@pytest.mark.parametrize("dist", ["normal", "ties", "zeros", "range"])
def test_sizes_and_distributions(S, dist):
    rows = 24 if S <= 8192 else 6
    rng = np.random.default_rng(S)
    s = _case(S + len(dist), rows, S, dist)
    lens = torch.from_numpy(rng.integers(0, S + 2, size=rows).astype(np.int32))
    cur = torch.from_numpy(np.array([rng.integers(-1, max(int(n), 1) + 1) for n in lens],
                                    np.int32))
    for topk in sorted({1, 2, 64, 512, max(S // 3, 1), S + 5}):
        run_and_check(s, cur, topk, lens, label="S%d %s k%d" % (S, dist, topk))


@pytest.mark.parametrize("S", [1000, 5000, 12000])
@pytest.mark.parametrize("dist", ["normal", "ties", "range"])
def test_two_workgroups_per_cu(S, dist):
    # More rows than CUs: the variant that keeps 16 keys per lane within 64
    # VGPRs (two workgroups per CU) for 4, 8 and 16 keys per lane.
    rows = 300
    rng = np.random.default_rng(S + 7)
    s = _case(S + 3 * len(dist), rows, S, dist)
    lens = torch.from_numpy(rng.integers(0, S + 2, size=rows).astype(np.int32))
    cur = torch.from_numpy(np.array([rng.integers(-1, max(int(n), 1) + 1) for n in lens],
                                    np.int32))
    for topk in (64, 512):
        run_and_check(s, cur, topk, lens, label="rows300 S%d %s k%d" % (S, dist, topk))


def _bin_case(seed, rows, S, m, tied):
    """Rows whose threshold falls in one bin of the first pass (12 or 13 bits) holding
    exactly m keys: 100 keys in [4, 4.5), m keys in [1, 1.0625) (distinct, or
    drawn from m // 8 + 1 values when tied), the rest negative; positions
    shuffled per row."""
    g = torch.Generator().manual_seed(seed)
    out = torch.empty((rows, S))
    for r in range(rows):
        hi = 4.0 + 0.5 * torch.rand(100, generator=g)
        if tied:
            nv = m // 8 + 1
            mid = 1.0 + (0.06 / nv) * torch.randint(0, nv, (m,), generator=g).float()
        else:
            mid = 1.0 + 0.06 * torch.rand(m, generator=g)
        lo = -1.0 - torch.rand(S - 100 - m, generator=g)
        row = torch.cat([hi, mid, lo])
        out[r] = row[torch.randperm(S, generator=g)]
    return out.float()


@pytest.mark.parametrize("m", [1, 3, 100, 1023, 1024, 1025, 4096, 4097])
@pytest.mark.parametrize("tied", [False, True])
def test_threshold_bin_sizes(m, tied):
    # The threshold bin is ranked directly up to 1024 keys, takes two more
    # radix passes over its LDS list up to 4096, and over the registers
    # beyond: every path, with the threshold at the bin's first, middle and
    # last key.
    # 12-bit first pass (8192 and 4400 columns) and 13-bit (12000 columns)
    for rows, S in ((8, 8192), (8, 12000), (260, 4400 if m <= 4096 else 8192), (260, 12000)):
        if rows == 260 and m not in (1, 1024, 1025, 4096, 4097):
            continue
        s = _bin_case(m + 31 * tied + rows, rows, S, m, tied)
        cur = torch.full((rows,), -1, dtype=torch.int32)
        for need in sorted({1, (m + 1) // 2, m}):
            run_and_check(s, cur, 100 + need, None,
                          label="bin m%d %s rows%d need%d" % (m, "tied" if tied else "distinct",
                                                             rows, need))


@pytest.mark.parametrize("rows,S", [(600, 32768), (1100, 5000)])
def test_more_rows_than_resident_workgroups(rows, S):
    # More rows than the chip holds workgroups at once (256 with 32 keys per
    # lane, 512 with at most 16): later rows start as earlier ones retire.
    rng = np.random.default_rng(rows)
    s = _case(rows + S, rows, S, "normal")
    lens = torch.from_numpy(rng.integers(0, S + 2, size=rows).astype(np.int32))
    cur = torch.from_numpy(np.array([rng.integers(-1, max(int(n), 1) + 1) for n in lens],
                                    np.int32))
    run_and_check(s, cur, 512, lens, label="loop rows%d S%d" % (rows, S))
    run_and_check(s, cur, 64, None, label="loop rows%d S%d no lengths" % (rows, S))


def test_no_lengths_all_columns():
    s = _case(3, 32, 3000, "normal")
    cur = torch.arange(32, dtype=torch.int32) * 90
    run_and_check(s, cur, 300, None, label="no lengths")


def test_strided_scores():
    big = _case(4, 16, 5000, "ties")
    s = big[:, 100:4196]                      # row stride 5000
    lens = torch.full((16,), 4000, dtype=torch.int32)
    cur = torch.full((16,), 3999, dtype=torch.int32)
    out = B.sda_select_regions(big.to(DEV)[:, 100:4196], cur.to(DEV), 512,
                               topk_lengths=lens.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.select_regions(np.ascontiguousarray(s.numpy()), cur.numpy(), 512, lens.numpy())
    assert np.array_equal(out.cpu().numpy(), ref)


def test_output_row_stride_and_untouched_padding_columns():
    s = _case(5, 8, 1024, "normal")
    cur = torch.full((8,), 100, dtype=torch.int32)
    buf = torch.full((8, 80), -9, dtype=torch.int32, device=DEV)
    B.sda_select_regions(s.to(DEV), cur.to(DEV), 64, out=buf[:, 8:72])
    torch.cuda.synchronize()
    ref = oracle.select_regions(s.numpy(), cur.numpy(), 64)
    b = buf.cpu().numpy()
    assert np.array_equal(b[:, 8:72], ref)
    assert (b[:, :8] == -9).all() and (b[:, 72:] == -9).all()


@pytest.mark.parametrize("name", ["select-decode", "select-large"])
@pytest.mark.parametrize("dist", ["normal", "ties"])
def test_full_size_workloads(name, dist):
    w = gen.SELECT_WORKLOADS[name]
    inp = gen.make_select_inputs(w, device=DEV, dist=dist)
    got = B.sda_select_regions(inp.scores, inp.current, w.topk, topk_lengths=inp.topk_lengths)
    torch.cuda.synchronize()
    ref = oracle.select_regions(inp.scores.cpu().numpy(), inp.current.cpu().numpy(), w.topk,
                                inp.topk_lengths.cpu().numpy())
    assert np.array_equal(got.cpu().numpy(), ref)


def test_selection_feeds_decode():
    # the selected regions drive sda_decode at 8-token regions: same output as
    # the oracle decode over the oracle's selection
    from oracle.hostprep import host_problem
    w = gen.Workload("sel-decode", requests=4, query_len=1, groups=2, heads=16, block=64,
                     pages_per_req=32, R=64, kv="bf16", pos_lo=600, pos_hi=2047, gated=True,
                     splits=1, region_tokens=8, seed=77)
    inp = gen.make_inputs(w, device=DEV)
    S = w.pages_per_req * w.block // 8
    cur = (inp.positions // 8).to(torch.int32)
    lens = (cur + 1).to(torch.int32)
    scores = torch.randn((w.rows, S), device=DEV)
    regions = B.sda_select_regions(scores, cur, w.R, topk_lengths=lens)
    out = torch.empty_like(inp.query)
    B.sda_decode(inp.query, inp.cache, regions, inp.block_table, inp.positions, inp.active, out,
                 scale=inp.scale, splits=1, gate=inp.gate, region_tokens=8)
    torch.cuda.synchronize()
    ref_regions = oracle.select_regions(scores.cpu().numpy(), cur.cpu().numpy(), w.R,
                                        lens.cpu().numpy())
    assert np.array_equal(regions.cpu().numpy(), ref_regions)
    hp = host_problem(inp.query, inp.cache, torch.from_numpy(ref_regions), inp.block_table,
                      inp.positions, inp.active, scale=inp.scale, region_tokens=8, gate=inp.gate)
    ref = oracle.decode(hp)
    err = np.abs(out.float().cpu().numpy() - ref)
    assert err.max() <= 1.5e-2 and err.mean() <= 1e-3
