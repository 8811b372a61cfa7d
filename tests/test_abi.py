"""C-ABI contract of libsda.so, on the host (no kernel is launched here)."""
import ctypes
import os
import re

import pytest
import torch

from sparse_paged_decode_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="sda.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(sda_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"sda_decode", "sda_splits", "sda_workspace_bytes", "sda_status_string",
            "sda_abi_version", "sda_args_size", "sda_swa_decode", "sda_swa_plan",
            "sda_select_regions", "sda_select_args_size", "sda_indexer_logits",
            "sda_logits_args_size", "sda_device_compute_units", "sda_decode_kernels",
            "sda_swa_args_size"} <= set(names)
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_struct_size():
    lib = B.lib()
    assert lib.sda_abi_version() == B.ABI_VERSION
    assert lib.sda_args_size() == ctypes.sizeof(B.DecodeArgs)
    assert lib.sda_swa_args_size() == ctypes.sizeof(B.SwaArgs)
    assert lib.sda_select_args_size() == ctypes.sizeof(B.SelectArgs)
    assert lib.sda_logits_args_size() == ctypes.sizeof(B.LogitsArgs)


def _table(name):
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", name)):
        line = line.split("#")[0].strip()
        if line:
            rows.append(tuple(int(x) for x in line.split()))
    return rows


@pytest.mark.parametrize("rows,splits", _table("splits_mi355x.txt"))
def test_split_heuristic_table(rows, splits):
    assert B.sda_splits(rows) == splits


def test_workspace_bytes():
    # [row order + row bins: 2*rows int32][partials + log-sum-exps when
    # splits > 1], each area rounded up to 256 bytes
    assert B.sda_workspace_bytes(256, 16, 1) == 2048
    assert B.sda_workspace_bytes(1000, 16, 1) == 8192
    assert B.sda_workspace_bytes(0, 16, 1) == 0
    n = 256 * 2 * 16 * 193 * 4
    assert B.sda_workspace_bytes(256, 16, 2) == 2048 + (n + 255) // 256 * 256
    assert B.sda_workspace_bytes(3, 5, 7) == 256 + (3 * 7 * 5 * 193 * 4 + 255) // 256 * 256
    assert B.sda_workspace_bytes(-1, 16, 2) == 0
    assert B.sda_workspace_bytes(4, 17, 2) == 0
    assert B.sda_workspace_bytes(4, 16, 0) == 0


def test_status_strings():
    for code in (0, -1, -2, -3, -4, 99):
        assert isinstance(B.status_string(code), str) and B.status_string(code)


# A fully valid argument block with fake (never dereferenced) device pointers.
def _valid_args(**over):
    a = B.DecodeArgs()
    a.rows, a.heads, a.groups, a.query_len, a.block, a.R, a.region_tokens = 8, 16, 4, 1, 64, 32, 0
    a.query, a.q_row_stride, a.q_head_stride = 0x100000, 16 * 192, 192
    a.output, a.o_row_stride, a.o_head_stride = 0x200000, 16 * 192, 192
    a.cache, a.kv_dtype = 0x300000, B.SDA_KV_BF16
    a.c_page_stride, a.c_group_stride, a.c_token_stride = 4 * 64 * 384, 64 * 384, 384
    a.regions, a.regions_row_stride = 0x400000, 32
    a.block_table, a.table_row_stride = 0x500000, 512
    a.positions, a.active = 0x600000, 0x700000
    a.scale, a.splits, a.clear_inactive = 0.07, 1, 1
    a.k_scale = a.v_scale = None
    a.gate = None
    a.workspace, a.workspace_bytes = None, 0
    for k, v in over.items():
        setattr(a, k, v)
    return a


INVALID = [
    dict(heads=0), dict(heads=17), dict(groups=0), dict(query_len=0), dict(block=0),
    dict(R=-1), dict(splits=0), dict(region_tokens=-1), dict(kv_dtype=2),
    dict(region_tokens=48),                    # does not divide block 64
    dict(rows=6),                              # not a multiple of groups * query_len
    dict(kv_dtype=B.SDA_KV_FP8_E4M3),          # FP8 without scales
    dict(kv_dtype=B.SDA_KV_FP8_E4M3, k_scale=0x800000),
    dict(query=None), dict(output=None), dict(cache=None), dict(block_table=None),
    dict(positions=None), dict(active=None), dict(regions=None),
    dict(rows=-4),
]

UNSUPPORTED = [
    dict(R=2049), dict(splits=257, workspace=0x900000, workspace_bytes=1 << 40),
    dict(query=0x100008), dict(q_head_stride=196), dict(q_row_stride=16 * 192 + 4),
    dict(cache=0x300008), dict(c_token_stride=388), dict(c_page_stride=4 * 64 * 384 + 4),
    dict(output=0x200002), dict(o_head_stride=193),
]


@pytest.mark.parametrize("over", INVALID, ids=[str(o) for o in INVALID])
def test_invalid_arguments_are_rejected(over):
    assert B.sda_decode_raw(_valid_args(**over)) == B.SDA_ERR_INVALID


@pytest.mark.parametrize("over", UNSUPPORTED, ids=[str(o) for o in UNSUPPORTED])
def test_unsupported_arguments_are_rejected(over):
    assert B.sda_decode_raw(_valid_args(**over)) == B.SDA_ERR_UNSUPPORTED


def test_workspace_checks():
    need = B.sda_workspace_bytes(8, 16, 4)
    assert B.sda_decode_raw(_valid_args(splits=4)) == B.SDA_ERR_WORKSPACE
    assert B.sda_decode_raw(_valid_args(splits=4, workspace=0x900000,
                                        workspace_bytes=need - 1)) == B.SDA_ERR_WORKSPACE
    assert B.sda_decode_raw(_valid_args(splits=4, workspace=0x900004,
                                        workspace_bytes=need)) == B.SDA_ERR_WORKSPACE
    # splits == 1: the workspace is optional, but one that is given must hold
    # the row order and be aligned
    need1 = B.sda_workspace_bytes(8, 16, 1)
    assert need1 == 256
    assert B.sda_decode_raw(_valid_args(splits=1, workspace=0x900000,
                                        workspace_bytes=need1 - 1)) == B.SDA_ERR_WORKSPACE
    assert B.sda_decode_raw(_valid_args(splits=1, workspace=0x900008,
                                        workspace_bytes=need1)) == B.SDA_ERR_WORKSPACE


def test_null_args_and_zero_rows():
    assert B.lib().sda_decode(None, None) == B.SDA_ERR_INVALID
    # rows == 0 returns OK without launching, even with null buffers
    a = _valid_args(rows=0, query=None, output=None, regions=None, positions=None, active=None)
    assert B.sda_decode_raw(a) == B.SDA_OK
    # ... but the shape contract is still checked first
    assert B.sda_decode_raw(_valid_args(rows=0, heads=17)) == B.SDA_ERR_INVALID


@pytest.mark.parametrize("over", INVALID + UNSUPPORTED + [dict(splits=4)],
                         ids=[str(o) for o in INVALID + UNSUPPORTED] + ["no workspace"])
def test_kernel_report_validates_like_decode(over):
    # sda_decode_kernels returns sda_decode's status and reports no kernels
    a = _valid_args(**over)
    rc, bits = B.sda_decode_kernels_raw(a)
    assert rc == B.sda_decode_raw(a) and rc != B.SDA_OK
    assert bits == 0


def test_kernel_report_edges():
    kernels = ctypes.c_int(7)
    assert B.lib().sda_decode_kernels(None, None, ctypes.byref(kernels)) == B.SDA_ERR_INVALID
    assert kernels.value == 0
    assert B.lib().sda_decode_kernels(ctypes.byref(_valid_args()), None, None) == B.SDA_ERR_INVALID
    a = _valid_args(rows=0, query=None, output=None, regions=None, positions=None, active=None)
    assert B.sda_decode_kernels_raw(a) == (B.SDA_OK, 0)
    # a valid call needs the device's CU count: without a device it fails as
    # sda_decode does, before any launch
    if not torch.cuda.is_available():
        assert B.sda_decode_kernels_raw(_valid_args()) == (B.SDA_ERR_LAUNCH, 0)


def test_fp8_scale_pointers_required_only_for_fp8():
    # bf16 with no scales is fine up to the launch; FP8 needs both (checked above).
    a = _valid_args(kv_dtype=B.SDA_KV_FP8_E4M3, k_scale=0x800000, v_scale=None)
    assert B.sda_decode_raw(a) == B.SDA_ERR_INVALID


def test_rows_limit():
    assert B.sda_decode_raw(_valid_args(rows=16777216, groups=1)) == B.SDA_ERR_UNSUPPORTED


# ---- sliding-window entry point ---------------------------------------------

@pytest.mark.parametrize("tokens,groups,heads,qlen,window,pack,splits",
                         _table("swa_plan_mi355x.txt"))
def test_swa_plan_table(tokens, groups, heads, qlen, window, pack, splits):
    # the table is worked for MI355X's 256 compute units, passed explicitly
    # (the page's swa_decode_plan takes the device's SM count the same way)
    assert B.sda_swa_plan(tokens, groups, heads, qlen, window, compute_units=256) == (pack,
                                                                                     splits)
    assert B.lib().sda_swa_plan(tokens, groups, heads, qlen, 256, window, None) == splits


@pytest.mark.parametrize("cus,splits", [(256, 4), (128, 2), (64, 1), (512, 8), (1024, 8)])
def test_swa_plan_follows_compute_units(cus, splits):
    # 16 requests x 4 groups = 64 workgroups, window 1024 (64 chunks): double
    # while 64 * splits * 2 <= cus and 64 >= 16 * splits (the chunk rule
    # holds 1024 CUs at 8).
    assert B.sda_swa_plan(16, 4, 16, 1, 1024, compute_units=cus) == (1, splits)


def test_device_compute_units_without_a_device():
    # No GPU in this process (or an out-of-range id): 0, never a guess.
    assert B.sda_device_compute_units(1 << 20) == 0


def _valid_swa(**over):
    a = B.SwaArgs()
    a.tokens, a.heads, a.groups, a.query_len, a.block, a.window = 8, 16, 4, 2, 64, 1024
    a.query, a.q_token_stride, a.q_head_stride = 0x100000, 64 * 192, 192
    a.output, a.o_token_stride, a.o_head_stride = 0x200000, 64 * 192, 192
    a.cache = 0x300000
    a.c_page_stride, a.c_group_stride, a.c_token_stride = 4 * 64 * 384, 64 * 384, 384
    a.block_table, a.table_row_stride = 0x500000, 128
    a.seq_lens = 0x600000
    a.scale, a.splits = 0.07, 1
    a.gate, a.gate_token_stride, a.gate_head_stride = 0x700000, 64, 1
    a.workspace, a.workspace_bytes = None, 0
    for k, v in over.items():
        setattr(a, k, v)
    return a


SWA_INVALID = [
    dict(heads=0), dict(heads=17), dict(groups=0), dict(query_len=0), dict(block=0),
    dict(window=0), dict(splits=0), dict(tokens=-2), dict(tokens=7),   # 7 % query_len 2
    dict(query=None), dict(output=None), dict(cache=None), dict(block_table=None),
    dict(seq_lens=None),
    dict(pack=-1), dict(pack=3),                      # max pack is min(2, 16 // 16) = 1
    dict(heads=4, pack=3),                            # > query_len 2
]

SWA_UNSUPPORTED = [
    dict(block=24),                                   # not a multiple of 16
    dict(block=16, window=2048 * 16),                 # page list beyond SDA_MAX_R
    dict(block=16, heads=8, pack=2, window=32736),    # + pack - 1 crosses the limit
    dict(splits=257, workspace=0x900000, workspace_bytes=1 << 40),
    dict(tokens=4194304, groups=4, query_len=1),      # rows beyond SDA_MAX_ROWS
    dict(query=0x100008), dict(q_head_stride=196), dict(q_token_stride=64 * 192 + 4),
    dict(cache=0x300008), dict(c_token_stride=388), dict(c_group_stride=64 * 384 + 4),
    dict(output=0x200002), dict(o_head_stride=193), dict(o_token_stride=64 * 192 + 1),
]


@pytest.mark.parametrize("over", SWA_INVALID, ids=[str(o) for o in SWA_INVALID])
def test_swa_invalid_arguments_are_rejected(over):
    assert B.sda_swa_decode_raw(_valid_swa(**over)) == B.SDA_ERR_INVALID


@pytest.mark.parametrize("over", SWA_UNSUPPORTED, ids=[str(o) for o in SWA_UNSUPPORTED])
def test_swa_unsupported_arguments_are_rejected(over):
    assert B.sda_swa_decode_raw(_valid_swa(**over)) == B.SDA_ERR_UNSUPPORTED


def test_swa_workspace_and_empty_batch():
    assert B.lib().sda_swa_decode(None, None) == B.SDA_ERR_INVALID
    need = B.sda_workspace_bytes(32, 16, 4)
    assert B.sda_swa_decode_raw(_valid_swa(splits=4)) == B.SDA_ERR_WORKSPACE
    assert B.sda_swa_decode_raw(_valid_swa(splits=4, workspace=0x900000,
                                           workspace_bytes=need - 1)) == B.SDA_ERR_WORKSPACE
    a = _valid_swa(tokens=0, query=None, output=None, seq_lens=None)
    assert B.sda_swa_decode_raw(a) == B.SDA_OK
    assert B.sda_swa_decode_raw(_valid_swa(tokens=0, heads=17)) == B.SDA_ERR_INVALID


def test_swa_pack_limit_edges():
    # (window + pack + 14) // block + 2 <= 2048 with block 16: the largest
    # window is 32736 at pack 1 and 32735 at pack 2.  splits = 2 with no
    # workspace makes an accepted shape stop at the workspace check, so no
    # kernel is ever launched on the fake pointers.
    for pack, window in ((1, 32736), (2, 32735)):
        rc = B.sda_swa_decode_raw(_valid_swa(block=16, heads=8, pack=pack, window=window,
                                             splits=2))
        assert rc == B.SDA_ERR_WORKSPACE, (pack, window, rc)


# ---- region selection entry point --------------------------------------------

def _valid_select(**over):
    a = B.SelectArgs()
    a.rows, a.num_regions, a.topk = 8, 4096, 512
    a.scores, a.scores_row_stride = 0x100000, 4096
    a.current, a.topk_lengths = 0x200000, 0x300000
    a.regions, a.regions_row_stride = 0x400000, 512
    for k, v in over.items():
        setattr(a, k, v)
    return a


SELECT_INVALID = [dict(rows=-1), dict(num_regions=-1), dict(topk=-1), dict(regions_row_stride=511),
                  dict(current=None), dict(regions=None), dict(scores=None),
                  dict(scores=0x100002), dict(current=0x200001), dict(regions=0x400003),
                  dict(topk_lengths=0x300002)]
SELECT_UNSUPPORTED = [dict(num_regions=32769), dict(rows=4194304), dict(rows=16777216)]


@pytest.mark.parametrize("over", SELECT_INVALID, ids=[str(o) for o in SELECT_INVALID])
def test_select_invalid_arguments_are_rejected(over):
    assert B.sda_select_regions_raw(_valid_select(**over)) == B.SDA_ERR_INVALID


@pytest.mark.parametrize("over", SELECT_UNSUPPORTED, ids=[str(o) for o in SELECT_UNSUPPORTED])
def test_select_unsupported_arguments_are_rejected(over):
    assert B.sda_select_regions_raw(_valid_select(**over)) == B.SDA_ERR_UNSUPPORTED


def test_select_empty_calls_launch_nothing():
    assert B.lib().sda_select_regions(None, None) == B.SDA_ERR_INVALID
    assert B.sda_select_regions_raw(_valid_select(rows=0, scores=None, current=None,
                                                  regions=None)) == B.SDA_OK
    assert B.sda_select_regions_raw(_valid_select(topk=0, regions_row_stride=0)) == B.SDA_OK
    # one row needs no row stride
    assert B.sda_select_regions_raw(_valid_select(rows=1, regions_row_stride=0, topk=0)) == \
        B.SDA_OK


# ---- indexer logits entry point -----------------------------------------------

def _valid_logits(**over):
    a = B.LogitsArgs()
    a.rows, a.heads, a.groups, a.query_len = 8, 8, 4, 1
    a.regions_per_page, a.num_regions, a.region_tokens = 8, 4096, 8
    a.query, a.q_row_stride, a.q_head_stride = 0x100000, 8 * 256, 256
    a.weights, a.w_row_stride = 0x200000, 8
    a.summaries, a.s_page_stride, a.s_region_stride = 0x300000, 8 * 256, 256
    a.summary_scales, a.ss_page_stride = 0x400000, 8
    a.block_table, a.table_row_stride = 0x500000, 512
    a.positions = 0x600000
    a.scores, a.scores_row_stride = 0x700000, 4096
    a.current = a.topk_lengths = None
    for k, v in over.items():
        setattr(a, k, v)
    return a


LOGITS_INVALID = [dict(heads=0), dict(heads=3), dict(heads=32), dict(groups=0), dict(query_len=0),
                  dict(regions_per_page=0), dict(num_regions=-1), dict(region_tokens=0),
                  dict(rows=6), dict(rows=-4), dict(query=None), dict(weights=None),
                  dict(summaries=None), dict(summary_scales=None), dict(block_table=None),
                  dict(positions=None), dict(scores=None), dict(weights=0x200002),
                  dict(current=0x800001), dict(table_cols=-1), dict(table_cols=513),
                  dict(scores=0x700002)]
LOGITS_UNSUPPORTED = [dict(heads=16, query_len=2), dict(query=0x100008),
                      dict(q_head_stride=264), dict(s_region_stride=260),
                      dict(summaries=0x300004), dict(rows=16777216 * 4, groups=4),
                      dict(num_regions=65535 * 256 + 1, scores_row_stride=65535 * 256 + 4)]


@pytest.mark.parametrize("over", LOGITS_INVALID, ids=[str(o) for o in LOGITS_INVALID])
def test_logits_invalid_arguments_are_rejected(over):
    assert B.sda_indexer_logits_raw(_valid_logits(**over)) == B.SDA_ERR_INVALID


@pytest.mark.parametrize("over", LOGITS_UNSUPPORTED, ids=[str(o) for o in LOGITS_UNSUPPORTED])
def test_logits_unsupported_arguments_are_rejected(over):
    assert B.sda_indexer_logits_raw(_valid_logits(**over)) == B.SDA_ERR_UNSUPPORTED


def test_logits_empty_calls_launch_nothing():
    assert B.lib().sda_indexer_logits(None, None) == B.SDA_ERR_INVALID
    assert B.sda_indexer_logits_raw(_valid_logits(rows=0, query=None)) == B.SDA_OK
    assert B.sda_indexer_logits_raw(_valid_logits(num_regions=0, scores=None)) == B.SDA_OK


def test_probe_library_exports_its_header():
    import ctypes
    from sparse_paged_decode_02_amd import build as sda_build
    names = _declared_functions("sda_probe.h")
    assert names == ["sda_probe_args_size", "sda_probe_gather", "sda_probe_valu"]
    lib = ctypes.CDLL(sda_build.PROBE_LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_valu_probe_validates_before_launching():
    # Every call here is rejected, or has nothing to launch, before any HIP call.
    import ctypes
    from sparse_paged_decode_02_amd import build as sda_build
    lib = ctypes.CDLL(sda_build.PROBE_LIB)
    lib.sda_probe_valu.restype = ctypes.c_int
    lib.sda_probe_valu.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
    dummy = ctypes.c_void_p(16)  # never dereferenced: each call returns first
    assert lib.sda_probe_valu(0, 0, 100, None, None) == B.SDA_OK
    assert lib.sda_probe_valu(0, 1, 100, None, None) == B.SDA_ERR_INVALID
    assert lib.sda_probe_valu(0, -1, 100, dummy, None) == B.SDA_ERR_INVALID
    assert lib.sda_probe_valu(0, 1, -1, dummy, None) == B.SDA_ERR_INVALID
    assert lib.sda_probe_valu(3, 1, 100, dummy, None) == B.SDA_ERR_INVALID
    assert lib.sda_probe_valu(-1, 1, 100, dummy, None) == B.SDA_ERR_INVALID
