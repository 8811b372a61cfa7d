"""Binding-side checks the C ABI cannot make because it sees only pointers
and strides: dtypes and shapes, a block table with fewer rows than the
request count that the row count implies, and a gate smaller than the rows
and heads read from it, are refused before anything reaches the device."""
import pytest
import torch

from sparse_paged_decode_02_amd import binding as B


def _decode_tensors(requests, table_rows):
    G, heads, block = 2, 4, 16
    rows = requests * G
    return dict(
        query=torch.zeros((rows, heads, 192), dtype=torch.bfloat16),
        cache=torch.zeros((4, G, block, 384), dtype=torch.bfloat16),
        regions=torch.zeros((rows, 2), dtype=torch.int32),
        block_table=torch.zeros((table_rows, 2), dtype=torch.int32),
        positions=torch.zeros(rows, dtype=torch.int32),
        active=torch.ones(rows, dtype=torch.uint8),
        output=torch.zeros((rows, heads, 192), dtype=torch.bfloat16))


def test_decode_refuses_short_block_table():
    t = _decode_tensors(requests=4, table_rows=3)
    with pytest.raises(B.SdaError) as e:
        B.sda_decode(t["query"], t["cache"], t["regions"], t["block_table"], t["positions"],
                     t["active"], t["output"], scale=1.0, splits=1, row_order=False)
    assert e.value.status == B.SDA_ERR_INVALID and "block_table" in str(e.value)


def test_swa_refuses_short_block_table():
    G, heads, tokens = 2, 4, 4
    with pytest.raises(B.SdaError) as e:
        B.sda_swa_decode(torch.zeros((tokens, G * heads, 192), dtype=torch.bfloat16),
                         torch.zeros((4, G, 64, 384), dtype=torch.bfloat16),
                         torch.zeros((tokens - 1, 4), dtype=torch.int32),
                         torch.full((tokens - 1,), 10, dtype=torch.int32),
                         torch.zeros((tokens, G * heads, 192), dtype=torch.bfloat16),
                         scale=1.0, window=8, query_len=1, splits=1)
    assert e.value.status == B.SDA_ERR_INVALID and "block_table" in str(e.value)


@pytest.mark.parametrize("query_len,table_rows", [(1, 3), (2, 1)])
def test_logits_refuses_short_block_table(query_len, table_rows):
    # 8 rows at 2 groups: 4 requests with one query token each, 2 with two.
    # A caller that passes query_len=1 for two-token requests asks for twice
    # the table rows it has; that is refused here.
    rows, heads = 8, 8
    with pytest.raises(B.SdaError) as e:
        B.sda_indexer_logits(torch.zeros((rows, heads, 256), dtype=torch.uint8),
                             torch.zeros((rows, heads), dtype=torch.float32),
                             torch.zeros((4, 8, 256), dtype=torch.uint8),
                             torch.zeros((4, 8), dtype=torch.float32),
                             torch.zeros((table_rows, 4), dtype=torch.int32),
                             torch.zeros(rows, dtype=torch.int32),
                             groups=2, num_regions=32, query_len=query_len)
    assert e.value.status == B.SDA_ERR_INVALID and "block_table" in str(e.value)


def _call(t, **kw):
    B.sda_decode(t["query"], t["cache"], t["regions"], t["block_table"], t["positions"],
                 t["active"], t["output"], scale=1.0, splits=1, row_order=False, **kw)


@pytest.mark.parametrize("gate_shape", [(3, 8), (4, 7)])
def test_decode_refuses_small_gate(gate_shape):
    t = _decode_tensors(requests=4, table_rows=4)  # 8 rows = 4 tokens x 2 groups, 4 heads
    with pytest.raises(B.SdaError) as e:
        _call(t, gate=torch.zeros(gate_shape, dtype=torch.bfloat16))
    assert e.value.status == B.SDA_ERR_INVALID and "gate" in str(e.value)


@pytest.mark.parametrize("bad", ["query_dtype", "head_dim", "output_shape", "query_stride",
                                 "cache_width", "cache_dtype", "regions_rows",
                                 "regions_dtype", "positions_len", "active_dtype",
                                 "scale_dtype", "gate_dtype"])
def test_decode_refuses_malformed_tensors(bad):
    t = _decode_tensors(requests=2, table_rows=2)
    kw = {}
    rows = t["query"].shape[0]
    if bad == "query_dtype":
        t["query"] = t["query"].float()
    elif bad == "head_dim":
        t["query"] = torch.zeros((rows, 4, 128), dtype=torch.bfloat16)
        t["output"] = torch.zeros((rows, 4, 128), dtype=torch.bfloat16)
    elif bad == "output_shape":
        t["output"] = torch.zeros((rows, 3, 192), dtype=torch.bfloat16)
    elif bad == "query_stride":
        t["query"] = torch.zeros((rows, 4, 384), dtype=torch.bfloat16)[..., ::2]
    elif bad == "cache_width":
        t["cache"] = torch.zeros((4, 2, 16, 256), dtype=torch.bfloat16)
    elif bad == "cache_dtype":
        t["cache"] = torch.zeros((4, 2, 16, 384), dtype=torch.float16)
    elif bad == "regions_rows":
        t["regions"] = torch.zeros((rows + 1, 2), dtype=torch.int32)
    elif bad == "regions_dtype":
        t["regions"] = torch.zeros((rows, 2), dtype=torch.int64)
    elif bad == "positions_len":
        t["positions"] = torch.zeros(rows - 1, dtype=torch.int32)
    elif bad == "active_dtype":
        t["active"] = torch.ones(rows, dtype=torch.int32)
    elif bad == "scale_dtype":
        t["cache"] = torch.zeros((4, 2, 16, 384), dtype=torch.uint8)
        kw = dict(k_scale=torch.ones(1, dtype=torch.float64), v_scale=torch.ones(1))
    elif bad == "gate_dtype":
        kw = dict(gate=torch.zeros((rows // 2, 8), dtype=torch.float32))
    with pytest.raises(B.SdaError) as e:
        _call(t, **kw)
    assert e.value.status == B.SDA_ERR_INVALID


@pytest.mark.parametrize("shape,dtype", [((3, 64), torch.float32), ((4, 32), torch.float32),
                                         ((4, 64), torch.float16)])
def test_logits_refuses_mismatched_scores(shape, dtype):
    # 4 rows (2 requests x 2 groups), 64 score columns requested
    q = torch.zeros((4, 8, 256), dtype=torch.uint8)
    with pytest.raises(B.SdaError) as e:
        B.sda_indexer_logits(q, torch.zeros((4, 8)), torch.zeros((8, 8, 256), dtype=torch.uint8),
                             torch.zeros((8, 8)), torch.zeros((2, 4), dtype=torch.int32),
                             torch.zeros(4, dtype=torch.int32), groups=2, num_regions=64,
                             scores=torch.zeros(shape, dtype=dtype))
    assert e.value.status == B.SDA_ERR_INVALID and "scores" in str(e.value)


def test_errors_name_their_call():
    # A wrapper's own argument checks name the call that refused them.
    with pytest.raises(B.SdaError) as e:
        B.sda_select_regions(torch.zeros((4, 16), dtype=torch.float64),
                             torch.zeros(4, dtype=torch.int32), 4)
    assert e.value.call == "sda_select_regions"
    assert str(e.value).startswith("sda_select_regions failed (%d)" % B.SDA_ERR_INVALID)
    with pytest.raises(B.SdaError) as e:
        B.sda_indexer_logits(torch.zeros((4, 8, 256), dtype=torch.float32), torch.zeros((4, 8)),
                             torch.zeros((8, 8, 256), dtype=torch.uint8), torch.zeros((8, 8)),
                             torch.zeros((2, 4), dtype=torch.int32),
                             torch.zeros(4, dtype=torch.int32), groups=2, num_regions=64)
    assert str(e.value).startswith("sda_indexer_logits failed")


# --- every tensor the library dereferences must be on the query's GPU --------
def test_decode_refuses_host_tensors():
    # Well-formed shapes on the host: refused before the C call (a host
    # pointer reaching a kernel would fault the device).
    t = _decode_tensors(requests=2, table_rows=2)
    with pytest.raises(B.SdaError) as e:
        _call(t)
    assert e.value.status == B.SDA_ERR_INVALID and "GPU" in str(e.value)


def test_swa_select_logits_refuse_host_tensors():
    G, heads, tokens = 2, 4, 4
    with pytest.raises(B.SdaError) as e:
        B.sda_swa_decode(torch.zeros((tokens, G * heads, 192), dtype=torch.bfloat16),
                         torch.zeros((4, G, 64, 384), dtype=torch.bfloat16),
                         torch.zeros((tokens, 4), dtype=torch.int32),
                         torch.full((tokens,), 10, dtype=torch.int32),
                         torch.zeros((tokens, G * heads, 192), dtype=torch.bfloat16),
                         scale=1.0, window=8, query_len=1, splits=1)
    assert e.value.status == B.SDA_ERR_INVALID and "GPU" in str(e.value)
    with pytest.raises(B.SdaError) as e:
        B.sda_select_regions(torch.zeros((4, 16)), torch.zeros(4, dtype=torch.int32), 4)
    assert e.value.status == B.SDA_ERR_INVALID and "GPU" in str(e.value)
    with pytest.raises(B.SdaError) as e:
        B.sda_indexer_logits(torch.zeros((4, 8, 256), dtype=torch.uint8), torch.zeros((4, 8)),
                             torch.zeros((8, 8, 256), dtype=torch.uint8), torch.zeros((8, 8)),
                             torch.zeros((2, 4), dtype=torch.int32),
                             torch.zeros(4, dtype=torch.int32), groups=2, num_regions=64)
    assert e.value.status == B.SDA_ERR_INVALID and "GPU" in str(e.value)


class _OnDevice:
    """Stand-in for a tensor on a given device (no GPU needed to test the
    rule itself)."""

    def __init__(self, device: str):
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"


@pytest.mark.parametrize("name,where", [("k_scale", "cpu"), ("gate", "cpu"),
                                        ("workspace", "cuda:1"), ("out", "cpu")])
def test_check_device_names_the_stray_tensor(name, where):
    ref = _OnDevice("cuda:0")
    others = {"cache": _OnDevice("cuda:0"), "v_scale": None, name: _OnDevice(where)}
    with pytest.raises(B.SdaError) as e:
        B.check_device(ref, **others)
    assert e.value.status == B.SDA_ERR_INVALID and name in str(e.value)
    B.check_device(ref, cache=_OnDevice("cuda:0"), v_scale=None)  # all on the GPU: fine


@pytest.mark.gpu
@pytest.mark.parametrize("stray", ["k_scale", "gate"])
def test_decode_refuses_host_scale_or_gate_gpu(stray):
    dev = "cuda:0"
    t = {k: v.to(dev) for k, v in _decode_tensors(requests=2, table_rows=2).items()}
    kw = {}
    if stray == "k_scale":
        t["cache"] = torch.zeros((4, 2, 16, 384), dtype=torch.uint8, device=dev)
        kw = dict(k_scale=torch.tensor([0.05]), v_scale=torch.tensor([0.04], device=dev))
    else:
        kw = dict(gate=torch.zeros((2, 8), dtype=torch.bfloat16))
    with pytest.raises(B.SdaError) as e:
        _call(t, **kw)
    assert e.value.status == B.SDA_ERR_INVALID and stray in str(e.value)
