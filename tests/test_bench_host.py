"""Host logic of bench.py (CPU): the one-GPU refusal, the algorithmic byte
counts the roofline divides by, and the counter-traffic lookup that ties a
profile summary to the kernel source it was measured on."""
import os
import subprocess
import sys

import numpy as np

import bench
from sparse_paged_decode_02_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _brute_force_tokens(w, positions, regions, active):
    """Visible selected tokens, one token at a time: slot by slot, token t of
    region id is counted iff id >= 0 and t <= the row's position."""
    n = 0
    for r in range(w.rows):
        if not active[r]:
            continue
        for rid in regions[r]:
            if rid < 0:
                continue
            for i in range(w.rt):
                if rid * w.rt + i <= positions[r]:
                    n += 1
    return n


def test_algorithmic_bytes_match_a_token_count():
    for k, kw in ((2, dict(requests=3, pages_per_req=24, pos_lo=100, pos_hi=1500)),
                  (3, dict(requests=4, pages_per_req=16, pos_lo=10, pos_hi=1023, R=12)),
                  (4, dict(requests=3, pages_per_req=16, pos_lo=40, pos_hi=510)),
                  (6, dict(requests=2, pages_per_req=16, pos_lo=7, pos_hi=1023, R=40))):
        w = gen.scaled(gen.WORKLOADS[k], **kw)
        idx = gen.draw_indices(w)
        got, tokens = bench.algorithmic_bytes(w, idx.positions, idx.regions, idx.active)
        want_tokens = _brute_force_tokens(w, idx.positions, idx.regions, idx.active)
        assert tokens == want_tokens
        e = 1 if w.kv == "fp8" else 2
        nact = int((idx.active != 0).sum())
        assert got == want_tokens * 384 * e + nact * w.heads * 384 + w.rows * w.heads * 384


def test_swa_algorithmic_bytes_count_each_window_token_once():
    w = gen.SWA_WORKLOADS["swa-mtp"]
    lens = np.array([1, 3, 4, 5, 1025, 8192] + [2000] * (w.requests - 6))
    got, tokens = bench.swa_algorithmic_bytes(w, lens)
    want = 0
    for L in lens:
        union = set()
        for j in range(w.query_len):
            p = L - w.query_len + j
            union.update(t for t in range(max(0, p - w.window + 1), p + 1) if t >= 0)
        want += len(union) * w.groups
    assert tokens == want
    assert got == want * 384 * 2 + 2 * w.rows * w.heads * 384


def test_traffic_is_read_only_for_the_profiled_kernel_and_split_count(tmp_path, monkeypatch):
    # A summary names the kernel source hash and split count it was measured
    # on; any other source or split count reads as no measurement (None).
    prof = tmp_path / "profiles"
    prof.mkdir()

    def summary(name, sha, splits, traffic):
        (prof / ("split_kernel_%s.md" % name)).write_text(
            "# x\n\n    kernel_sha256_16 = %s\n    splits = %d\n\n"
            "    traffic_bytes_per_launch = %d\n" % (sha, splits, traffic))

    summary("current", bench.kernel_hash(), 1, 12345)
    summary("stale", "0123456789abcdef", 1, 777)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("current", 1) == 12345
    assert bench.load_traffic("current", 2) is None
    assert bench.load_traffic("stale", 1) is None
    assert bench.load_traffic("missing", 1) is None


def test_record_keeps_the_one_line_contract():
    # The fields and units of the JSON line, and the roofline arithmetic:
    # achieved = algorithmic bytes per launch / average launch time.
    class A:
        steps, warmup = 10, 2
    rec = bench.record(A, value=6000.0, wall=10 * 61e-6, launch_avg_ms=0.0605,
                       launch_ms=np.full(10, 0.061), bytes_per_launch=379478208.0, rows=256,
                       dtype="bf16", config={"workload": "x"}, kernel="k", traffic=380000000)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in rec
    assert rec["metric"] == bench.METRIC and rec["unit"] == "GB/s" and rec["n_gpus"] == 1
    assert rec["higher_is_better"] is True and rec["vs_baseline"] is None
    assert rec["data"] == "synthetic" and rec["config"] == {"workload": "x"}
    assert abs(rec["ms_per_step"] - 0.061) < 1e-9
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert abs(roof["achieved"] - 379478208.0 / 60.5e-6 / 1e9) < 0.01
    assert abs(roof["frac"] - roof["achieved"] / 8000.0) < 1e-4
    assert roof["traffic"] == 380000000
    assert abs(rec["rows_per_s"] - 256 * 10 / (10 * 61e-6)) < 1.0


def _parsed(*argv):
    class A:
        pass
    a = A()
    a.config, a.also = 5, None
    for k, v in zip(argv[::2], argv[1::2]):
        setattr(a, k, v)
    return a


def test_default_headline_is_the_largest_workload_with_the_others_after_it():
    # The driver runs bench.py with no --config: the headline is workload 5
    # (large-batch FP8, the largest), and workloads 2-4 follow in the same run.
    r = subprocess.run([sys.executable, "-c",
                        "import sys, bench; sys.argv = ['bench.py', '--help']; bench.main()"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert "default 5" in r.stdout
    assert bench.parse_also(_parsed()) == [2, 3, 4]
    assert bench.parse_also(_parsed("config", 2)) == []
    assert bench.parse_also(_parsed("also", "")) == []
    assert bench.parse_also(_parsed("config", 3, "also", "2,4")) == [2, 4]
    assert gen.WORKLOADS[5].rows == max(w.rows for k, w in gen.WORKLOADS.items() if k <= 5)


def test_summary_keeps_each_workloads_roofline():
    class A:
        steps, warmup = 10, 2
    rec = bench.record(A, value=6000.0, wall=1e-3, launch_avg_ms=0.1, launch_ms=np.full(10, 0.1),
                       bytes_per_launch=6e8, rows=512, dtype="bf16", config={"workload": "y"},
                       kernel="k", traffic=None)
    s = bench.summary_of(rec)
    assert s["roofline"] == rec["roofline"] and s["config"] == {"workload": "y"}
    assert "metric" not in s and "n_gpus" not in s


def test_host_threads_use_every_usable_core_up_to_the_stated_share(monkeypatch):
    avail = len(os.sched_getaffinity(0))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    assert bench.host_threads()[0] == avail
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    n, why = bench.host_threads()
    assert n == 1 and "OMP_NUM_THREADS=1" in why
    monkeypatch.setenv("OMP_NUM_THREADS", str(avail + 5))
    assert bench.host_threads()[0] == avail


def test_probe_blocks_are_each_rows_visible_regions():
    # Byte offsets of the blocks the gather probe reads, against a slot-by-slot
    # walk: every visible region (id >= 0, first token <= position) of every
    # active row, in slot order, at page * ps + g * gs + (t0 % block) * ts.
    for k, kw in ((2, dict(requests=3, pages_per_req=24, pos_lo=100, pos_hi=1500)),
                  (4, dict(requests=3, pages_per_req=16, pos_lo=40, pos_hi=510)),
                  (7, dict(requests=2, pages_per_req=16, pos_lo=7, pos_hi=1023, R=40))):
        w = gen.scaled(gen.WORKLOADS[k], **kw)
        idx = gen.draw_indices(w)
        e = 1 if w.kv == "fp8" else 2
        strides = (w.groups * w.block * 384 + 64, w.block * 384 + 32, 384 + 16)
        offs, start = bench.probe_blocks(w, strides, idx.positions, idx.regions, idx.active,
                                         idx.block_table)
        want, wstart = [], [0]
        for r in range(w.rows):
            if idx.active[r]:
                req, g = r // (w.groups * w.query_len), r % w.groups
                for rid in idx.regions[r]:
                    if rid >= 0 and rid * w.rt <= idx.positions[r]:
                        t0 = int(rid) * w.rt
                        page = int(idx.block_table[req, t0 // w.block])
                        want.append((page * strides[0] + g * strides[1]
                                     + (t0 % w.block) * strides[2]) * e)
            wstart.append(len(want))
        assert offs.tolist() == want and start.tolist() == wstart
