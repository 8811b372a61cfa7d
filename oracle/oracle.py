"""ctypes wrapper around the fp64 C oracle (``sda_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module.  The HIP library never imports or calls it,
and it imports nothing from the HIP package.

Inputs are numpy arrays on the host.  bf16 tensors are passed as their uint16
bit patterns and FP8 e4m3 tensors as their uint8 bytes; the oracle decodes
both itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sda_oracle.c")
_LIB = os.path.join(_HERE, "libsda_oracle.so")

KV_BF16 = 0
KV_FP8_E4M3 = 1
DIM = 192


_LIB_SAN = os.path.join(_HERE, "libsda_oracle_san.so")
# Sanitizer flags for the checked build: every report aborts the process.
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def sanitized() -> bool:
    """True when the checked build is selected (SDA_ORACLE_SANITIZE=1).  The
    process must then have the ASan and UBSan runtimes preloaded."""
    return os.environ.get("SDA_ORACLE_SANITIZE", "") == "1"


def build(force: bool = False, sanitize: bool | None = None) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math).  ``sanitize``
    (default: ``sanitized()``) builds the AddressSanitizer +
    UndefinedBehaviorSanitizer variant instead, libsda_oracle_san.so."""
    if sanitize is None:
        sanitize = sanitized()
    lib_path = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(lib_path) or \
            os.path.getmtime(lib_path) < os.path.getmtime(_SRC):
        tmp = lib_path + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-Wall", "-Wextra"] + (SANITIZE_FLAGS if sanitize else []) +
            ["-o", tmp, _SRC, "-lm"])
        os.replace(tmp, lib_path)
    return lib_path


class _Problem(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("heads", ctypes.c_int32), ("groups", ctypes.c_int32),
        ("query_len", ctypes.c_int32), ("block", ctypes.c_int32), ("R", ctypes.c_int32),
        ("region_tokens", ctypes.c_int32),
        ("query", ctypes.c_void_p), ("q_row_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("cache", ctypes.c_void_p), ("kv_dtype", ctypes.c_int32),
        ("c_page_stride", ctypes.c_int64), ("c_group_stride", ctypes.c_int64),
        ("c_token_stride", ctypes.c_int64), ("num_pages", ctypes.c_int64),
        ("regions", ctypes.c_void_p), ("regions_row_stride", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("table_row_stride", ctypes.c_int64),
        ("table_cols", ctypes.c_int64),
        ("positions", ctypes.c_void_p), ("active", ctypes.c_void_p),
        ("scale", ctypes.c_float), ("clear_inactive", ctypes.c_int32),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("gate", ctypes.c_void_p), ("gate_row_stride", ctypes.c_int64),
        ("gate_head_stride", ctypes.c_int64),
    ]


class _SwaProblem(ctypes.Structure):
    _fields_ = [
        ("tokens", ctypes.c_int32), ("heads", ctypes.c_int32), ("groups", ctypes.c_int32),
        ("query_len", ctypes.c_int32), ("block", ctypes.c_int32), ("window", ctypes.c_int32),
        ("query", ctypes.c_void_p), ("q_row_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("cache", ctypes.c_void_p),
        ("c_page_stride", ctypes.c_int64), ("c_group_stride", ctypes.c_int64),
        ("c_token_stride", ctypes.c_int64), ("num_pages", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("table_row_stride", ctypes.c_int64),
        ("table_cols", ctypes.c_int64),
        ("seq_lens", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("gate", ctypes.c_void_p), ("gate_row_stride", ctypes.c_int64),
        ("gate_head_stride", ctypes.c_int64),
    ]


class _LogitsProblem(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("heads", ctypes.c_int32), ("groups", ctypes.c_int32),
        ("query_len", ctypes.c_int32), ("rpb", ctypes.c_int32), ("num_regions", ctypes.c_int32),
        ("region_tokens", ctypes.c_int32),
        ("query", ctypes.c_void_p), ("q_row_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("weights", ctypes.c_void_p), ("w_row_stride", ctypes.c_int64),
        ("summaries", ctypes.c_void_p), ("s_page_stride", ctypes.c_int64),
        ("s_region_stride", ctypes.c_int64),
        ("scales", ctypes.c_void_p), ("sc_page_stride", ctypes.c_int64),
        ("num_pages", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("table_row_stride", ctypes.c_int64),
        ("table_cols", ctypes.c_int64),
        ("positions", ctypes.c_void_p),
    ]


_lib = None
_lib_lock = threading.Lock()


def lib():
    global _lib
    with _lib_lock:
        if _lib is None:
            l = ctypes.CDLL(build())
            l.sdo_bf16_to_double.restype = ctypes.c_double
            l.sdo_bf16_to_double.argtypes = [ctypes.c_uint16]
            l.sdo_e4m3_to_double.restype = ctypes.c_double
            l.sdo_e4m3_to_double.argtypes = [ctypes.c_uint8]
            l.sdo_f32_to_bf16_bits.restype = ctypes.c_uint16
            l.sdo_f32_to_bf16_bits.argtypes = [ctypes.c_float]
            l.sdo_gate_value.restype = ctypes.c_float
            l.sdo_gate_value.argtypes = [ctypes.c_uint16]
            l.sdo_splits_pages.restype = ctypes.c_int
            l.sdo_splits_pages.argtypes = [ctypes.c_int]
            l.sdo_decode.restype = ctypes.c_int
            l.sdo_decode.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p,
                                     ctypes.c_int, ctypes.c_int]
            l.sdo_decode_split.restype = ctypes.c_int
            l.sdo_decode_split.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
            l.sdo_select_regions.restype = ctypes.c_int
            l.sdo_select_regions.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
            l.sdo_indexer_logits.restype = ctypes.c_int
            l.sdo_indexer_logits.argtypes = [ctypes.POINTER(_LogitsProblem), ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_int]
            l.sdo_swa_decode.restype = ctypes.c_int
            l.sdo_swa_decode.argtypes = [ctypes.POINTER(_SwaProblem), ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_int]
            _lib = l
    return _lib


def bf16_to_double(bits: int) -> float:
    return lib().sdo_bf16_to_double(bits)


def e4m3_to_double(bits: int) -> float:
    return lib().sdo_e4m3_to_double(bits)


def f32_to_bf16_bits(x: float) -> int:
    return lib().sdo_f32_to_bf16_bits(x)


def gate_value(bits: int) -> float:
    return lib().sdo_gate_value(bits)


def splits_pages(rows: int) -> int:
    return lib().sdo_splits_pages(rows)


@dataclass
class HostProblem:
    """Host copies of every input, in the layouts the C ABI takes.

    query: uint16 [rows, heads, 192] (bf16 bits, any strides with unit inner)
    cache: uint16 (bf16 bits) or uint8 (e4m3) [pages, G, block, 384]
    regions: int32 [rows, R]; block_table: int32 [requests, cols]
    positions: int32 [rows]; active: uint8 [rows]; gate: uint16 or None
    """
    query: np.ndarray
    cache: np.ndarray
    regions: np.ndarray
    block_table: np.ndarray
    positions: np.ndarray
    active: np.ndarray
    scale: float
    query_len: int = 1
    region_tokens: int = 0
    clear_inactive: bool = True
    k_scale: float = 1.0
    v_scale: float = 1.0
    gate: np.ndarray | None = None


def _strides(a: np.ndarray) -> tuple:
    return tuple(s // a.itemsize for s in a.strides)


def _problem(hp: HostProblem) -> _Problem:
    q, c = hp.query, hp.cache
    assert q.dtype == np.uint16 and q.ndim == 3 and q.shape[2] == DIM and q.strides[2] == 2
    assert c.ndim == 4 and c.shape[3] == 2 * DIM and c.strides[3] == c.itemsize
    assert c.dtype in (np.uint16, np.uint8)
    assert hp.regions.dtype == np.int32 and hp.regions.strides[1] == 4
    assert hp.block_table.dtype == np.int32 and hp.block_table.strides[1] == 4
    assert hp.positions.dtype == np.int32 and hp.positions.flags.c_contiguous
    assert hp.active.dtype == np.uint8 and hp.active.flags.c_contiguous
    rows, heads, _ = q.shape
    p = _Problem()
    p.rows, p.heads, p.groups = rows, heads, c.shape[1]
    p.query_len, p.block, p.R = hp.query_len, c.shape[2], hp.regions.shape[1]
    p.region_tokens = hp.region_tokens
    p.query = q.ctypes.data
    p.q_row_stride, p.q_head_stride = _strides(q)[0], _strides(q)[1]
    p.cache = c.ctypes.data
    p.kv_dtype = KV_BF16 if c.dtype == np.uint16 else KV_FP8_E4M3
    cs = _strides(c)
    p.c_page_stride, p.c_group_stride, p.c_token_stride = cs[0], cs[1], cs[2]
    p.num_pages = c.shape[0]
    p.regions = hp.regions.ctypes.data
    p.regions_row_stride = _strides(hp.regions)[0]
    p.block_table = hp.block_table.ctypes.data
    p.table_row_stride = _strides(hp.block_table)[0]
    p.table_cols = hp.block_table.shape[1]
    p.positions = hp.positions.ctypes.data
    p.active = hp.active.ctypes.data
    p.scale = hp.scale
    p.clear_inactive = 1 if hp.clear_inactive else 0
    p.k_scale, p.v_scale = hp.k_scale, hp.v_scale
    if hp.gate is not None:
        assert hp.gate.dtype == np.uint16
        p.gate = hp.gate.ctypes.data
        p.gate_row_stride, p.gate_head_stride = _strides(hp.gate)
    else:
        p.gate = None
        p.gate_row_stride = p.gate_head_stride = 0
    return p


def _check_rc(rc: int) -> None:
    if rc != 0:
        raise RuntimeError({-1: "bad arguments", -2: "block-table column out of range",
                            -3: "page id not present in the host cache",
                            -4: "out of memory"}.get(rc, "error %d" % rc))


def decode(hp: HostProblem, out: np.ndarray | None = None, rows=None,
           splits: int | None = None, threads: int = 1) -> np.ndarray:
    """fp64 reference output [rows, heads, 192].

    ``out``: fp64 array to write into (rows left untouched by the semantics,
    i.e. inactive rows with clear_inactive off, keep its contents); default is
    a NaN-filled array.  ``rows``: optional iterable of row ids to compute
    (others stay untouched).  ``splits``: use the split/merge organisation
    with that many splits instead of the direct definition.  ``threads``:
    host threads, each taking whole rows.
    """
    nrows, heads = hp.query.shape[0], hp.query.shape[1]
    if out is None:
        out = np.full((nrows, heads, DIM), np.nan)
    assert out.dtype == np.float64 and out.shape == (nrows, heads, DIM) and out.flags.c_contiguous
    p = _problem(hp)
    l = lib()
    row_list = list(range(nrows)) if rows is None else [int(r) for r in rows]
    row_bytes = heads * DIM * 8

    def run(rs):
        for r in rs:
            ptr = out.ctypes.data + r * row_bytes
            if splits is None:
                rc = l.sdo_decode(ctypes.byref(p), ptr, r, r + 1)
            else:
                rc = l.sdo_decode_split(ctypes.byref(p), splits, ptr, r, r + 1)
            _check_rc(rc)

    if threads <= 1 or len(row_list) < 2:
        run(row_list)
    else:
        parts = [row_list[i::threads] for i in range(threads)]
        errs = []

        def worker(rs):
            try:
                run(rs)
            except Exception as e:  # surfaced below
                errs.append(e)

        ts = [threading.Thread(target=worker, args=(rs,)) for rs in parts if rs]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        if errs:
            raise errs[0]
    return out


@dataclass
class SwaHostProblem:
    """Host copies of the gated sliding-window decode inputs.

    query: uint16 [tokens*G, heads, 192], the row view (row r is group r % G
    of token r // G); cache: uint16 [pages, G, block, 384] (bf16 bits);
    block_table: int32 [requests, cols]; seq_lens: int32 [requests];
    gate: uint16 [tokens, G*heads] or None.
    """
    query: np.ndarray
    cache: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    scale: float
    window: int
    query_len: int = 1
    gate: np.ndarray | None = None


def _swa_problem(hp: SwaHostProblem) -> _SwaProblem:
    q, c = hp.query, hp.cache
    assert q.dtype == np.uint16 and q.ndim == 3 and q.shape[2] == DIM and q.strides[2] == 2
    assert c.dtype == np.uint16 and c.ndim == 4 and c.shape[3] == 2 * DIM and c.strides[3] == 2
    assert hp.block_table.dtype == np.int32 and hp.block_table.strides[1] == 4
    assert hp.seq_lens.dtype == np.int32 and hp.seq_lens.flags.c_contiguous
    groups = c.shape[1]
    assert q.shape[0] % groups == 0
    p = _SwaProblem()
    p.tokens, p.heads, p.groups = q.shape[0] // groups, q.shape[1], groups
    p.query_len, p.block, p.window = hp.query_len, c.shape[2], hp.window
    p.query = q.ctypes.data
    p.q_row_stride, p.q_head_stride = _strides(q)[0], _strides(q)[1]
    p.cache = c.ctypes.data
    cs = _strides(c)
    p.c_page_stride, p.c_group_stride, p.c_token_stride = cs[0], cs[1], cs[2]
    p.num_pages = c.shape[0]
    p.block_table = hp.block_table.ctypes.data
    p.table_row_stride = _strides(hp.block_table)[0]
    p.table_cols = hp.block_table.shape[1]
    p.seq_lens = hp.seq_lens.ctypes.data
    p.scale = hp.scale
    if hp.gate is not None:
        assert hp.gate.dtype == np.uint16
        p.gate = hp.gate.ctypes.data
        p.gate_row_stride, p.gate_head_stride = _strides(hp.gate)
    else:
        p.gate = None
        p.gate_row_stride = p.gate_head_stride = 0
    return p


def swa_decode(hp: SwaHostProblem, rows=None, threads: int = 1) -> np.ndarray:
    """fp64 reference output [tokens*G, heads, 192] of the gated
    sliding-window decode (rows not listed in ``rows`` stay NaN)."""
    nrows, heads = hp.query.shape[0], hp.query.shape[1]
    out = np.full((nrows, heads, DIM), np.nan)
    p = _swa_problem(hp)
    l = lib()
    row_list = list(range(nrows)) if rows is None else [int(r) for r in rows]
    row_bytes = heads * DIM * 8

    def run(rs):
        for r in rs:
            _check_rc(l.sdo_swa_decode(ctypes.byref(p), out.ctypes.data + r * row_bytes, r, r + 1))

    if threads <= 1 or len(row_list) < 2:
        run(row_list)
    else:
        errs = []

        def worker(rs):
            try:
                run(rs)
            except Exception as e:  # surfaced below
                errs.append(e)

        ts = [threading.Thread(target=worker, args=(row_list[i::threads],))
              for i in range(threads) if row_list[i::threads]]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        if errs:
            raise errs[0]
    return out


def select_regions(scores: np.ndarray, current: np.ndarray, topk: int,
                   topk_lengths: np.ndarray | None = None) -> np.ndarray:
    """int32 [rows, topk]: the selected region ids of each row in ascending
    order, then -1 (see ``sdo_select_regions``).  ``scores``: float32
    [rows, S] (any row stride, unit inner stride)."""
    assert scores.dtype == np.float32 and scores.ndim == 2
    assert scores.strides[1] == 4 or scores.shape[1] <= 1
    rows, S = scores.shape
    cur = np.ascontiguousarray(current, dtype=np.int32)
    assert cur.shape == (rows,)
    lens = None if topk_lengths is None else np.ascontiguousarray(topk_lengths, dtype=np.int32)
    out = np.full((rows, topk), -7, dtype=np.int32)
    rs = scores.strides[0] // 4 if rows > 1 else S
    _check_rc(lib().sdo_select_regions(rows, S, topk, scores.ctypes.data, rs, cur.ctypes.data,
                                       None if lens is None else lens.ctypes.data,
                                       out.ctypes.data, topk))
    return out


@dataclass
class LogitsHostProblem:
    """Host copies of the decode indexer-logits inputs.

    query: uint8 e4m3 [rows, heads, 256]; weights: float32 [rows, heads];
    summaries: uint8 e4m3 [pages, rpb, 256]; scales: float32 [pages, rpb];
    block_table: int32 [requests, cols]; positions: int32 [rows].
    """
    query: np.ndarray
    weights: np.ndarray
    summaries: np.ndarray
    scales: np.ndarray
    block_table: np.ndarray
    positions: np.ndarray
    groups: int
    num_regions: int
    query_len: int = 1
    region_tokens: int = 8


def indexer_logits(hp: LogitsHostProblem, rows=None, threads: int = 1) -> np.ndarray:
    """fp64 scores [rows, num_regions] (rows not listed stay NaN)."""
    q, w, sm, sc = hp.query, hp.weights, hp.summaries, hp.scales
    assert q.dtype == np.uint8 and q.ndim == 3 and q.shape[2] == 256 and q.strides[2] == 1
    assert w.dtype == np.float32 and w.shape == q.shape[:2] and w.strides[1] == 4
    assert sm.dtype == np.uint8 and sm.ndim == 3 and sm.shape[2] == 256 and sm.strides[2] == 1
    assert sc.dtype == np.float32 and sc.shape == sm.shape[:2] and sc.strides[1] == 4
    bt = hp.block_table
    assert bt.dtype == np.int32 and bt.strides[1] == 4
    pos = np.ascontiguousarray(hp.positions, dtype=np.int32)
    p = _LogitsProblem()
    p.rows, p.heads, p.groups = q.shape[0], q.shape[1], hp.groups
    p.query_len, p.rpb, p.num_regions = hp.query_len, sm.shape[1], hp.num_regions
    p.region_tokens = hp.region_tokens
    p.query = q.ctypes.data
    p.q_row_stride, p.q_head_stride = q.strides[0], q.strides[1]
    p.weights = w.ctypes.data
    p.w_row_stride = w.strides[0] // 4
    p.summaries = sm.ctypes.data
    p.s_page_stride, p.s_region_stride = sm.strides[0], sm.strides[1]
    p.scales = sc.ctypes.data
    p.sc_page_stride = sc.strides[0] // 4
    p.num_pages = sm.shape[0]
    p.block_table = bt.ctypes.data
    p.table_row_stride = bt.strides[0] // 4
    p.table_cols = bt.shape[1]
    p.positions = pos.ctypes.data
    out = np.full((q.shape[0], hp.num_regions), np.nan)
    l = lib()
    row_list = list(range(q.shape[0])) if rows is None else [int(r) for r in rows]
    row_bytes = hp.num_regions * 8

    def run(rs):
        for r in rs:
            _check_rc(l.sdo_indexer_logits(ctypes.byref(p), out.ctypes.data + r * row_bytes,
                                           r, r + 1))

    if threads <= 1 or len(row_list) < 2:
        run(row_list)
    else:
        errs = []

        def worker(rs):
            try:
                run(rs)
            except Exception as e:  # surfaced below
                errs.append(e)

        ts = [threading.Thread(target=worker, args=(row_list[i::threads],))
              for i in range(threads) if row_list[i::threads]]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        if errs:
            raise errs[0]
    return out
