"""ctypes binding of libsda.so (see include/sda.h).

Argument marshalling only: tensors become device pointers and element
strides, and every step of the computation runs in the HIP library.  PyTorch
supplies device memory and the stream.  If libsda.so is missing, the first call
raises; nothing falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsda.so")

SDA_OK = 0
SDA_ERR_INVALID = -1
SDA_ERR_UNSUPPORTED = -2
SDA_ERR_WORKSPACE = -3
SDA_ERR_LAUNCH = -4
SDA_ERR_SCRATCH = -5
STATIC_SCRATCH_BYTES = 16 << 20
SDA_KV_BF16 = 0
SDA_KV_FP8_E4M3 = 1
SDA_KERNEL_ORDER = 1
SDA_KERNEL_SPLIT = 2
SDA_KERNEL_ROW_STREAM = 4
SDA_KERNEL_COMBINE = 8
ABI_VERSION = 8
HEAD_DIM = 192


class SdaError(RuntimeError):
    """A library call's sda_status, with the call it came from (argument
    checks shared by several calls name none)."""
    def __init__(self, status: int, message: str, call: str = ""):
        super().__init__("%s failed (%d): %s" % (call or "sda call", status, message))
        self.status = status
        self.call = call


class DecodeArgs(ctypes.Structure):
    """Mirror of ``sda_decode_args``; checked against sda_args_size()."""
    _fields_ = [
        ("rows", ctypes.c_int32), ("heads", ctypes.c_int32), ("groups", ctypes.c_int32),
        ("query_len", ctypes.c_int32), ("block", ctypes.c_int32), ("R", ctypes.c_int32),
        ("region_tokens", ctypes.c_int32),
        ("query", ctypes.c_void_p), ("q_row_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("output", ctypes.c_void_p), ("o_row_stride", ctypes.c_int64),
        ("o_head_stride", ctypes.c_int64),
        ("cache", ctypes.c_void_p), ("kv_dtype", ctypes.c_int32),
        ("c_page_stride", ctypes.c_int64), ("c_group_stride", ctypes.c_int64),
        ("c_token_stride", ctypes.c_int64),
        ("regions", ctypes.c_void_p), ("regions_row_stride", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("table_row_stride", ctypes.c_int64),
        ("positions", ctypes.c_void_p), ("active", ctypes.c_void_p),
        ("scale", ctypes.c_float), ("splits", ctypes.c_int32),
        ("clear_inactive", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("gate", ctypes.c_void_p), ("gate_row_stride", ctypes.c_int64),
        ("gate_head_stride", ctypes.c_int64),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class SwaArgs(ctypes.Structure):
    """Mirror of ``sda_swa_args``; checked against sda_swa_args_size()."""
    _fields_ = [
        ("tokens", ctypes.c_int32), ("heads", ctypes.c_int32), ("groups", ctypes.c_int32),
        ("query_len", ctypes.c_int32), ("block", ctypes.c_int32), ("window", ctypes.c_int32),
        ("pack", ctypes.c_int32),
        ("query", ctypes.c_void_p), ("q_token_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("output", ctypes.c_void_p), ("o_token_stride", ctypes.c_int64),
        ("o_head_stride", ctypes.c_int64),
        ("cache", ctypes.c_void_p),
        ("c_page_stride", ctypes.c_int64), ("c_group_stride", ctypes.c_int64),
        ("c_token_stride", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("table_row_stride", ctypes.c_int64),
        ("seq_lens", ctypes.c_void_p),
        ("scale", ctypes.c_float), ("splits", ctypes.c_int32),
        ("gate", ctypes.c_void_p), ("gate_token_stride", ctypes.c_int64),
        ("gate_head_stride", ctypes.c_int64),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class SelectArgs(ctypes.Structure):
    """Mirror of ``sda_select_args``; checked against sda_select_args_size()."""
    _fields_ = [
        ("rows", ctypes.c_int32), ("num_regions", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("scores", ctypes.c_void_p), ("scores_row_stride", ctypes.c_int64),
        ("current", ctypes.c_void_p), ("topk_lengths", ctypes.c_void_p),
        ("regions", ctypes.c_void_p), ("regions_row_stride", ctypes.c_int64),
    ]


class LogitsArgs(ctypes.Structure):
    """Mirror of ``sda_logits_args``; checked against sda_logits_args_size()."""
    _fields_ = [
        ("rows", ctypes.c_int32), ("heads", ctypes.c_int32), ("groups", ctypes.c_int32),
        ("query_len", ctypes.c_int32), ("regions_per_page", ctypes.c_int32),
        ("num_regions", ctypes.c_int32), ("region_tokens", ctypes.c_int32),
        ("query", ctypes.c_void_p), ("q_row_stride", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64),
        ("weights", ctypes.c_void_p), ("w_row_stride", ctypes.c_int64),
        ("summaries", ctypes.c_void_p), ("s_page_stride", ctypes.c_int64),
        ("s_region_stride", ctypes.c_int64),
        ("summary_scales", ctypes.c_void_p), ("ss_page_stride", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("table_row_stride", ctypes.c_int64),
        ("positions", ctypes.c_void_p),
        ("scores", ctypes.c_void_p), ("scores_row_stride", ctypes.c_int64),
        ("current", ctypes.c_void_p), ("topk_lengths", ctypes.c_void_p),
        ("table_cols", ctypes.c_int32),
    ]


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libsda.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    "libsda.so is not built (%s); run __graft_entry__.build() or "
                    "python -m sparse_paged_decode_02_amd.build" % LIB_PATH)
            l = ctypes.CDLL(LIB_PATH)
            l.sda_decode.restype = ctypes.c_int
            l.sda_decode.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
            l.sda_decode_kernels.restype = ctypes.c_int
            l.sda_decode_kernels.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p,
                                             ctypes.POINTER(ctypes.c_int)]
            l.sda_decode_static.restype = ctypes.c_int
            l.sda_decode_static.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
            l.sda_splits.restype = ctypes.c_int
            l.sda_splits.argtypes = [ctypes.c_int]
            l.sda_workspace_bytes.restype = ctypes.c_size_t
            l.sda_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
            l.sda_status_string.restype = ctypes.c_char_p
            l.sda_status_string.argtypes = [ctypes.c_int]
            l.sda_abi_version.restype = ctypes.c_int
            l.sda_abi_version.argtypes = []
            l.sda_args_size.restype = ctypes.c_size_t
            l.sda_args_size.argtypes = []
            l.sda_swa_decode.restype = ctypes.c_int
            l.sda_swa_decode.argtypes = [ctypes.POINTER(SwaArgs), ctypes.c_void_p]
            l.sda_swa_plan.restype = ctypes.c_int
            l.sda_swa_plan.argtypes = [ctypes.c_int] * 6 + [ctypes.POINTER(ctypes.c_int)]
            l.sda_device_compute_units.restype = ctypes.c_int
            l.sda_device_compute_units.argtypes = [ctypes.c_int]
            l.sda_swa_args_size.restype = ctypes.c_size_t
            l.sda_swa_args_size.argtypes = []
            l.sda_select_regions.restype = ctypes.c_int
            l.sda_select_regions.argtypes = [ctypes.POINTER(SelectArgs), ctypes.c_void_p]
            l.sda_select_args_size.restype = ctypes.c_size_t
            l.sda_select_args_size.argtypes = []
            l.sda_indexer_logits.restype = ctypes.c_int
            l.sda_indexer_logits.argtypes = [ctypes.POINTER(LogitsArgs), ctypes.c_void_p]
            l.sda_logits_args_size.restype = ctypes.c_size_t
            l.sda_logits_args_size.argtypes = []
            if l.sda_abi_version() != ABI_VERSION:
                raise RuntimeError("libsda.so ABI version %d, binding expects %d"
                                   % (l.sda_abi_version(), ABI_VERSION))
            if l.sda_args_size() != ctypes.sizeof(DecodeArgs):
                raise RuntimeError("sda_decode_args size mismatch: library %d, binding %d"
                                   % (l.sda_args_size(), ctypes.sizeof(DecodeArgs)))
            if l.sda_logits_args_size() != ctypes.sizeof(LogitsArgs):
                raise RuntimeError("sda_logits_args size mismatch: library %d, binding %d"
                                   % (l.sda_logits_args_size(), ctypes.sizeof(LogitsArgs)))
            if l.sda_select_args_size() != ctypes.sizeof(SelectArgs):
                raise RuntimeError("sda_select_args size mismatch: library %d, binding %d"
                                   % (l.sda_select_args_size(), ctypes.sizeof(SelectArgs)))
            if l.sda_swa_args_size() != ctypes.sizeof(SwaArgs):
                raise RuntimeError("sda_swa_args size mismatch: library %d, binding %d"
                                   % (l.sda_swa_args_size(), ctypes.sizeof(SwaArgs)))
            _lib = l
    return _lib


def sda_splits(rows: int) -> int:
    return int(lib().sda_splits(int(rows)))


def sda_workspace_bytes(rows: int, heads: int, splits: int) -> int:
    return int(lib().sda_workspace_bytes(int(rows), int(heads), int(splits)))


def status_string(status: int) -> str:
    return lib().sda_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else t.data_ptr()


def make_args(query, cache, regions, block_table, positions, active, output, *, scale,
              query_len=1, splits, clear_inactive=True, k_scale=None, v_scale=None,
              gate=None, region_tokens=0, workspace=None) -> DecodeArgs:
    """Fill ``sda_decode_args`` from tensors (no validation beyond the C side)."""
    a = DecodeArgs()
    rows, heads = query.shape[0], query.shape[1]
    a.rows, a.heads = rows, heads
    a.groups, a.query_len, a.block = cache.shape[1], int(query_len), cache.shape[2]
    a.R = regions.shape[1] if regions.dim() == 2 else 0
    a.region_tokens = int(region_tokens)
    a.query = _ptr(query)
    a.q_row_stride, a.q_head_stride = query.stride(0), query.stride(1)
    a.output = _ptr(output)
    a.o_row_stride, a.o_head_stride = output.stride(0), output.stride(1)
    a.cache = _ptr(cache)
    fp8 = cache.dtype in (torch.uint8, torch.float8_e4m3fn)
    a.kv_dtype = SDA_KV_FP8_E4M3 if fp8 else SDA_KV_BF16
    a.c_page_stride, a.c_group_stride, a.c_token_stride = (
        cache.stride(0), cache.stride(1), cache.stride(2))
    a.regions = _ptr(regions)
    a.regions_row_stride = regions.stride(0) if regions.dim() == 2 else 0
    a.block_table = _ptr(block_table)
    a.table_row_stride = block_table.stride(0)
    a.positions = _ptr(positions)
    a.active = _ptr(active)
    a.scale = float(scale)
    a.splits = int(splits)
    a.clear_inactive = 1 if clear_inactive else 0
    a.k_scale = _ptr(k_scale)
    a.v_scale = _ptr(v_scale)
    a.gate = _ptr(gate)
    if gate is not None:
        a.gate_row_stride, a.gate_head_stride = gate.stride(0), gate.stride(1)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return a


def check_device(ref, **tensors) -> None:
    """Every tensor the library dereferences must live on ``ref``'s GPU: the
    C ABI sees only pointers, and a host pointer reaching a kernel would fault
    the device.  ``None`` entries (optional arguments) are skipped."""
    if not ref.is_cuda:
        raise SdaError(SDA_ERR_INVALID, "tensors must be on a GPU (got %s)" % ref.device)
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != ref.device):
            raise SdaError(SDA_ERR_INVALID, "%s is on %s; every tensor must be on %s"
                           % (name, t.device, ref.device))


def check_tensors(query, cache, regions, block_table, positions, active, output,
                  k_scale, v_scale, gate):
    """dtype and shape checks the C ABI cannot make (it sees only pointers)."""
    if query.dtype != torch.bfloat16 or output.dtype != torch.bfloat16:
        raise SdaError(SDA_ERR_INVALID, "query and output must be bfloat16")
    if query.dim() != 3 or output.shape != query.shape or query.shape[2] != HEAD_DIM:
        raise SdaError(SDA_ERR_INVALID, "query/output must be [rows, heads, 192]")
    if query.stride(2) != 1 or output.stride(2) != 1:
        raise SdaError(SDA_ERR_INVALID, "query/output need unit stride in dim 2")
    if cache.dim() != 4 or cache.shape[3] != 2 * HEAD_DIM or cache.stride(3) != 1:
        raise SdaError(SDA_ERR_INVALID, "cache must be [pages, G, block, 384], unit last stride")
    if cache.dtype not in (torch.bfloat16, torch.uint8, torch.float8_e4m3fn):
        raise SdaError(SDA_ERR_INVALID, "cache must be bfloat16 or FP8 e4m3 (uint8 storage)")
    if regions.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise SdaError(SDA_ERR_INVALID, "regions and block_table must be int32")
    if regions.dim() != 2 or regions.shape[0] != query.shape[0] or (
            regions.shape[1] > 0 and regions.stride(1) != 1):
        raise SdaError(SDA_ERR_INVALID, "regions must be [rows, R] with unit inner stride")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise SdaError(SDA_ERR_INVALID, "block_table must be 2-D with unit inner stride")
    if positions.dtype != torch.int32 or not positions.is_contiguous() or \
            positions.numel() != query.shape[0]:
        raise SdaError(SDA_ERR_INVALID, "positions must be contiguous int32 [rows]")
    if active.dtype not in (torch.bool, torch.uint8) or not active.is_contiguous() or \
            active.numel() != query.shape[0]:
        raise SdaError(SDA_ERR_INVALID, "active must be contiguous bool/uint8 [rows]")
    for s in (k_scale, v_scale):
        if s is not None and (s.dtype != torch.float32 or s.numel() != 1):
            raise SdaError(SDA_ERR_INVALID, "k_scale/v_scale must be fp32 scalars")
    if gate is not None and (gate.dtype != torch.bfloat16 or gate.dim() != 2):
        raise SdaError(SDA_ERR_INVALID, "gate must be bfloat16 [tokens, G*heads]")


def check_table_rows(block_table, rows: int, rows_per_request: int) -> None:
    """The library derives the request count from the row count (rows per
    request = KV groups x query tokens) and sees only the table's row stride,
    so a table with too few rows would be read past its end: refuse it here."""
    if rows_per_request < 1 or rows % rows_per_request or block_table.dim() != 2:
        return  # the C side rejects these shapes itself
    need = rows // rows_per_request
    if block_table.shape[0] < need:
        raise SdaError(SDA_ERR_INVALID,
                       "block_table has %d rows; %d rows at %d per request need %d" % (
                           block_table.shape[0], rows, rows_per_request, need))


def check_gate_shape(gate, rows: int, groups: int, heads: int) -> None:
    """gate [tokens, groups * heads]: the library reads gate[r / groups,
    (r % groups) * heads + h] for every row r and head h, so a smaller gate
    would be read past its end: refuse it here."""
    if gate is None or groups < 1 or rows % groups or gate.dim() != 2:
        return  # absent, or a shape the other checks reject
    if gate.shape[0] < rows // groups or gate.shape[1] < groups * heads:
        raise SdaError(SDA_ERR_INVALID,
                       "gate is [%d, %d]; %d rows of %d heads in %d KV groups need "
                       "[%d, %d]" % (gate.shape[0], gate.shape[1], rows, heads, groups,
                                     rows // groups, groups * heads))


def _decode_call(query, cache, regions, block_table, positions, active, output, scale,
                 query_len, splits, clear_inactive, k_scale, v_scale, gate, region_tokens,
                 workspace, row_order, stream):
    """Checked sda_decode_args and stream handle for one decode call."""
    check_tensors(query, cache, regions, block_table, positions, active, output,
                  k_scale, v_scale, gate)
    rows, heads = query.shape[0], query.shape[1]
    check_table_rows(block_table, rows, cache.shape[1] * int(query_len))
    check_gate_shape(gate, rows, cache.shape[1], heads)
    check_device(query, cache=cache, regions=regions, block_table=block_table,
                 positions=positions, active=active, output=output, k_scale=k_scale,
                 v_scale=v_scale, gate=gate, workspace=workspace)
    if workspace is None and (splits > 1 or row_order) and rows > 0:
        nbytes = sda_workspace_bytes(rows, heads, splits)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=query.device)
    a = make_args(query, cache, regions, block_table, positions, active, output, scale=scale,
                  query_len=query_len, splits=splits, clear_inactive=clear_inactive,
                  k_scale=k_scale, v_scale=v_scale, gate=gate, region_tokens=region_tokens,
                  workspace=workspace)
    if stream is None:
        stream = torch.cuda.current_stream(query.device)
    # the workspace tensor must outlive the enqueue: keep it with the args
    return a, ctypes.c_void_p(stream.cuda_stream), workspace


def sda_decode(query, cache, regions, block_table, positions, active, output, *, scale,
               query_len=1, splits, clear_inactive=True, k_scale=None, v_scale=None,
               gate=None, region_tokens=0, workspace=None, row_order=True,
               stream=None) -> None:
    """Enqueue ``sda_decode`` on ``stream`` (default: torch's current stream).

    Argument names follow ``sparse_decode_attention`` on the page
    "vllm.models.step5.nvidia.ops.sparse_decode_attention".  ``workspace``: a
    device tensor of at least sda_workspace_bytes(rows, heads, splits) bytes;
    allocated here through torch when omitted, unless splits == 1 and
    ``row_order`` is false (no workspace: rows start in index order).
    """
    a, handle, _ws = _decode_call(query, cache, regions, block_table, positions, active, output,
                                  scale, query_len, splits, clear_inactive, k_scale, v_scale,
                                  gate, region_tokens, workspace, row_order, stream)
    rc = lib().sda_decode(ctypes.byref(a), handle)
    if rc != SDA_OK:
        raise SdaError(rc, status_string(rc), call="sda_decode")


def sda_decode_kernels(query, cache, regions, block_table, positions, active, output, *, scale,
                       query_len=1, splits, clear_inactive=True, k_scale=None, v_scale=None,
                       gate=None, region_tokens=0, workspace=None, row_order=True,
                       stream=None) -> int:
    """SDA_KERNEL_* bits of the kernels ``sda_decode`` with the same arguments
    would launch; nothing is launched."""
    a, handle, _ws = _decode_call(query, cache, regions, block_table, positions, active, output,
                                  scale, query_len, splits, clear_inactive, k_scale, v_scale,
                                  gate, region_tokens, workspace, row_order, stream)
    rc, bits = sda_decode_kernels_raw(a, handle)
    if rc != SDA_OK:
        raise SdaError(rc, status_string(rc), call="sda_decode_kernels")
    return bits


def sda_decode_static(query, cache, regions, block_table, positions, active, output, *,
                      scale, query_len=1, splits, clear_inactive=True, k_scale=None,
                      v_scale=None, gate=None, region_tokens=0, stream=None) -> None:
    """Enqueue ``sda_decode_static``: ``sda_decode`` with the library's static
    device scratch as its workspace, so that nothing is allocated, here or in
    the library.  Calls that overlap on one GPU share that scratch."""
    check_tensors(query, cache, regions, block_table, positions, active, output,
                  k_scale, v_scale, gate)
    rows, heads = query.shape[0], query.shape[1]
    check_table_rows(block_table, rows, cache.shape[1] * int(query_len))
    check_gate_shape(gate, rows, cache.shape[1], heads)
    check_device(query, cache=cache, regions=regions, block_table=block_table,
                 positions=positions, active=active, output=output, k_scale=k_scale,
                 v_scale=v_scale, gate=gate)
    a = make_args(query, cache, regions, block_table, positions, active, output, scale=scale,
                  query_len=query_len, splits=splits, clear_inactive=clear_inactive,
                  k_scale=k_scale, v_scale=v_scale, gate=gate, region_tokens=region_tokens)
    if stream is None:
        stream = torch.cuda.current_stream(query.device)
    rc = lib().sda_decode_static(ctypes.byref(a), ctypes.c_void_p(stream.cuda_stream))
    if rc != SDA_OK:
        raise SdaError(rc, status_string(rc), call="sda_decode_static")


def sda_decode_static_raw(args: DecodeArgs, stream_handle=None) -> int:
    """Call sda_decode_static on a prepared struct; returns the status code."""
    return int(lib().sda_decode_static(ctypes.byref(args), stream_handle))


def sda_decode_raw(args: DecodeArgs, stream_handle=None) -> int:
    """Call the C entry point on a prepared struct; returns the status code."""
    return int(lib().sda_decode(ctypes.byref(args), stream_handle))


def sda_decode_kernels_raw(args: DecodeArgs, stream_handle=None) -> tuple:
    """(status, SDA_KERNEL_* bits) of the kernels sda_decode would launch for
    a prepared struct; nothing is launched."""
    bits = ctypes.c_int(0)
    rc = int(lib().sda_decode_kernels(ctypes.byref(args), stream_handle, ctypes.byref(bits)))
    return rc, int(bits.value)


def sda_swa_plan(tokens: int, groups: int, heads: int, query_len: int, window: int,
                 compute_units: int = 0) -> tuple:
    """(pack, splits) the library picks for a sliding-window call on a device
    with ``compute_units`` CUs (0: the current device)."""
    pack = ctypes.c_int(0)
    splits = lib().sda_swa_plan(int(tokens), int(groups), int(heads), int(query_len),
                                int(compute_units), int(window), ctypes.byref(pack))
    return int(pack.value), int(splits)


def sda_device_compute_units(device: int = -1) -> int:
    """Compute units of HIP device ``device`` (-1: the current one); 0 if the
    runtime cannot report it."""
    return int(lib().sda_device_compute_units(int(device)))


def make_swa_args(query, cache, block_table, seq_lens, output, *, scale, window, query_len=1,
                  splits, pack=0, gate=None, workspace=None) -> SwaArgs:
    """Fill ``sda_swa_args`` from tensors (no validation beyond the C side).
    ``query``/``output``: [tokens, groups*heads, 192]; ``cache``: [pages,
    groups, block, 384]."""
    a = SwaArgs()
    groups = cache.shape[1]
    a.tokens, a.heads, a.groups = query.shape[0], query.shape[1] // groups, groups
    a.query_len, a.block, a.window = int(query_len), cache.shape[2], int(window)
    a.pack = int(pack)
    a.query = _ptr(query)
    a.q_token_stride, a.q_head_stride = query.stride(0), query.stride(1)
    a.output = _ptr(output)
    a.o_token_stride, a.o_head_stride = output.stride(0), output.stride(1)
    a.cache = _ptr(cache)
    a.c_page_stride, a.c_group_stride, a.c_token_stride = (
        cache.stride(0), cache.stride(1), cache.stride(2))
    a.block_table = _ptr(block_table)
    a.table_row_stride = block_table.stride(0)
    a.seq_lens = _ptr(seq_lens)
    a.scale = float(scale)
    a.splits = int(splits)
    a.gate = _ptr(gate)
    if gate is not None:
        a.gate_token_stride, a.gate_head_stride = gate.stride(0), gate.stride(1)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return a


def check_swa_tensors(query, cache, block_table, seq_lens, output, gate):
    """dtype and shape checks the C ABI cannot make (it sees only pointers)."""
    if query.dtype != torch.bfloat16 or output.dtype != torch.bfloat16:
        raise SdaError(SDA_ERR_INVALID, "query and output must be bfloat16")
    if query.dim() != 3 or output.shape != query.shape or query.shape[2] != HEAD_DIM:
        raise SdaError(SDA_ERR_INVALID, "query/output must be [tokens, heads, 192]")
    if query.stride(2) != 1 or output.stride(2) != 1:
        raise SdaError(SDA_ERR_INVALID, "query/output need unit stride in dim 2")
    if cache.dtype != torch.bfloat16 or cache.dim() != 4 or cache.shape[3] != 2 * HEAD_DIM \
            or cache.stride(3) != 1:
        raise SdaError(SDA_ERR_INVALID, "cache must be bfloat16 [pages, G, block, 384]")
    if query.shape[1] % cache.shape[1]:
        raise SdaError(SDA_ERR_INVALID, "query heads must be a multiple of the KV groups")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise SdaError(SDA_ERR_INVALID, "block_table must be int32 2-D, unit inner stride")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous() or \
            seq_lens.numel() != block_table.shape[0]:
        raise SdaError(SDA_ERR_INVALID, "seq_lens must be contiguous int32 [requests]")
    if gate is not None and (gate.dtype != torch.bfloat16 or gate.dim() != 2 or
                             gate.shape != query.shape[:2]):
        raise SdaError(SDA_ERR_INVALID, "gate must be bfloat16 [tokens, heads]")


def sda_swa_decode(query, cache, block_table, seq_lens, output, *, scale, window,
                   query_len=1, splits, pack=0, gate=None, workspace=None,
                   stream=None) -> None:
    """Enqueue ``sda_swa_decode`` (gated sliding-window decode) on ``stream``.

    Argument names follow ``swa_decode_gated`` as ``forward_with_headwise_gate``
    calls it on the page "vllm.models.step5.nvidia.sparse_attention", with the
    packed cache in place of its K and V views.  The workspace is allocated
    here through torch when omitted and splits > 1.
    """
    check_swa_tensors(query, cache, block_table, seq_lens, output, gate)
    check_table_rows(block_table, query.shape[0], int(query_len))
    check_device(query, cache=cache, block_table=block_table, seq_lens=seq_lens,
                 output=output, gate=gate, workspace=workspace)
    groups = cache.shape[1]
    rows, heads = query.shape[0] * groups, query.shape[1] // groups
    if workspace is None and splits > 1 and rows > 0:
        nbytes = sda_workspace_bytes(rows, heads, splits)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=query.device)
    a = make_swa_args(query, cache, block_table, seq_lens, output, scale=scale, window=window,
                      query_len=query_len, splits=splits, pack=pack, gate=gate,
                      workspace=workspace)
    if stream is None:
        stream = torch.cuda.current_stream(query.device)
    handle = ctypes.c_void_p(stream.cuda_stream)
    rc = lib().sda_swa_decode(ctypes.byref(a), handle)
    if rc != SDA_OK:
        raise SdaError(rc, status_string(rc), call="sda_swa_decode")


def sda_swa_decode_raw(args: SwaArgs, stream_handle=None) -> int:
    """Call sda_swa_decode on a prepared struct; returns the status code."""
    return int(lib().sda_swa_decode(ctypes.byref(args), stream_handle))


def make_select_args(scores, current, topk, out, topk_lengths=None) -> SelectArgs:
    """Fill ``sda_select_args`` from tensors (no validation beyond the C side)."""
    a = SelectArgs()
    a.rows, a.num_regions, a.topk = scores.shape[0], scores.shape[1], int(topk)
    a.scores = _ptr(scores)
    a.scores_row_stride = scores.stride(0)
    a.current = _ptr(current)
    a.topk_lengths = _ptr(topk_lengths)
    a.regions = _ptr(out)
    a.regions_row_stride = out.stride(0) if out.dim() == 2 else 0
    return a


def sda_select_regions(scores, current, topk, *, topk_lengths=None, out=None,
                       stream=None):
    """Enqueue ``sda_select_regions``; returns the int32 [rows, topk] regions.

    Argument names follow ``select_regions`` on the page "vllm.models.step5.
    nvidia.flashinfer_sparse" (``sort=False``)."""
    if scores.dtype != torch.float32 or scores.dim() != 2 or (
            scores.shape[1] > 1 and scores.stride(1) != 1):
        raise SdaError(SDA_ERR_INVALID, "scores must be float32 [rows, regions], unit inner stride",
                       call="sda_select_regions")
    rows = scores.shape[0]
    for t, name in ((current, "current"), (topk_lengths, "topk_lengths")):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or
                              t.numel() != rows):
            raise SdaError(SDA_ERR_INVALID, "%s must be contiguous int32 [rows]" % name,
                           call="sda_select_regions")
    if out is None:
        out = torch.empty((rows, int(topk)), dtype=torch.int32, device=scores.device)
    if out.dtype != torch.int32 or out.dim() != 2 or out.shape != (rows, int(topk)) or (
            topk > 1 and out.stride(1) != 1):
        raise SdaError(SDA_ERR_INVALID, "out must be int32 [rows, topk], unit inner stride",
                       call="sda_select_regions")
    check_device(scores, current=current, topk_lengths=topk_lengths, out=out)
    a = make_select_args(scores, current, topk, out, topk_lengths)
    if stream is None:
        stream = torch.cuda.current_stream(scores.device)
    handle = ctypes.c_void_p(stream.cuda_stream)
    rc = lib().sda_select_regions(ctypes.byref(a), handle)
    if rc != SDA_OK:
        raise SdaError(rc, status_string(rc), call="sda_select_regions")
    return out


def sda_select_regions_raw(args: SelectArgs, stream_handle=None) -> int:
    """Call sda_select_regions on a prepared struct; returns the status code."""
    return int(lib().sda_select_regions(ctypes.byref(args), stream_handle))


def make_logits_args(query, weights, summaries, summary_scales, block_table, positions, scores,
                     *, groups, query_len=1, region_tokens=8, current=None,
                     topk_lengths=None, table_cols=None) -> LogitsArgs:
    """Fill ``sda_logits_args`` from tensors.  e4m3 tensors are uint8 (or
    float8_e4m3fn) storage; their strides become bytes.  ``table_cols``:
    block_table's column count (None: its shape; 0: unknown, so only the
    scored regions' columns are read)."""
    a = LogitsArgs()
    a.rows, a.heads, a.groups, a.query_len = query.shape[0], query.shape[1], int(groups), \
        int(query_len)
    a.regions_per_page, a.num_regions = summaries.shape[1], scores.shape[1]
    a.region_tokens = int(region_tokens)
    a.query = _ptr(query)
    a.q_row_stride, a.q_head_stride = query.stride(0), query.stride(1)
    a.weights = _ptr(weights)
    a.w_row_stride = weights.stride(0)
    a.summaries = _ptr(summaries)
    a.s_page_stride, a.s_region_stride = summaries.stride(0), summaries.stride(1)
    a.summary_scales = _ptr(summary_scales)
    a.ss_page_stride = summary_scales.stride(0)
    a.block_table = _ptr(block_table)
    a.table_row_stride = block_table.stride(0)
    a.table_cols = block_table.shape[1] if table_cols is None else int(table_cols)
    a.positions = _ptr(positions)
    a.scores = _ptr(scores)
    a.scores_row_stride = scores.stride(0)
    a.current = _ptr(current)
    a.topk_lengths = _ptr(topk_lengths)
    return a


def sda_indexer_logits(query, weights, summaries, summary_scales, block_table, positions, *,
                       groups, num_regions, query_len=1, region_tokens=8, scores=None,
                       current=None, topk_lengths=None, table_cols=None, stream=None):
    """Enqueue ``sda_indexer_logits``; returns the fp32 [rows, num_regions] scores.

    Names follow ``decode_logits`` on the page "vllm.models.step5.nvidia.
    flashinfer_sparse" (query, weights, the per-page region summaries with
    their scales, table, positions).  ``table_cols``: as in make_logits_args."""
    e4 = (torch.uint8, torch.float8_e4m3fn)
    if query.dtype not in e4 or query.dim() != 3 or query.shape[2] != 256 or query.stride(2) != 1:
        raise SdaError(SDA_ERR_INVALID, "query must be e4m3 [rows, heads, 256]",
                       call="sda_indexer_logits")
    if summaries.dtype not in e4 or summaries.dim() != 3 or summaries.shape[2] != 256 or \
            summaries.stride(2) != 1:
        raise SdaError(SDA_ERR_INVALID, "summaries must be e4m3 [pages, regions_per_page, 256]",
                       call="sda_indexer_logits")
    if weights.dtype != torch.float32 or weights.shape != query.shape[:2] or (
            weights.shape[1] > 1 and weights.stride(1) != 1):
        raise SdaError(SDA_ERR_INVALID, "weights must be float32 [rows, heads]",
                       call="sda_indexer_logits")
    if summary_scales.dtype != torch.float32 or summary_scales.shape != summaries.shape[:2] or (
            summary_scales.shape[1] > 1 and summary_scales.stride(1) != 1):
        raise SdaError(SDA_ERR_INVALID, "summary_scales must be float32 [pages, regions_per_page]",
                       call="sda_indexer_logits")
    for t, name in ((block_table, "block_table"),):
        if t.dtype != torch.int32 or t.dim() != 2 or t.stride(1) != 1:
            raise SdaError(SDA_ERR_INVALID, "%s must be int32 2-D, unit inner stride" % name,
                           call="sda_indexer_logits")
    rows = query.shape[0]
    check_table_rows(block_table, rows, int(groups) * int(query_len))
    for t, name in ((positions, "positions"), (current, "current"),
                    (topk_lengths, "topk_lengths")):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or
                              t.numel() != rows):
            raise SdaError(SDA_ERR_INVALID, "%s must be contiguous int32 [rows]" % name,
                           call="sda_indexer_logits")
    if scores is None:
        scores = torch.empty((rows, int(num_regions)), dtype=torch.float32, device=query.device)
    if scores.dtype != torch.float32 or scores.dim() != 2 or \
            tuple(scores.shape) != (rows, int(num_regions)) or \
            (scores.shape[1] > 1 and scores.stride(1) != 1):
        raise SdaError(SDA_ERR_INVALID,
                       "scores must be float32 [rows, num_regions], unit inner stride",
                       call="sda_indexer_logits")
    check_device(query, weights=weights, summaries=summaries, summary_scales=summary_scales,
                 block_table=block_table, positions=positions, scores=scores, current=current,
                 topk_lengths=topk_lengths)
    a = make_logits_args(query, weights, summaries, summary_scales, block_table, positions,
                         scores, groups=groups, query_len=query_len, region_tokens=region_tokens,
                         current=current, topk_lengths=topk_lengths, table_cols=table_cols)
    if stream is None:
        stream = torch.cuda.current_stream(query.device)
    handle = ctypes.c_void_p(stream.cuda_stream)
    rc = lib().sda_indexer_logits(ctypes.byref(a), handle)
    if rc != SDA_OK:
        raise SdaError(rc, status_string(rc), call="sda_indexer_logits")
    return scores


def sda_indexer_logits_raw(args: LogitsArgs, stream_handle=None) -> int:
    """Call sda_indexer_logits on a prepared struct; returns the status code."""
    return int(lib().sda_indexer_logits(ctypes.byref(args), stream_handle))
