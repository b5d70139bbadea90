"""The Python binding rejects tensors that do not fit the cache's shape before anything reaches the library.

The C ABI receives bare pointers and cannot see a tensor's sizes, so a batch smaller than the cache's, a float16 or
too small output, or a short workspace would make the kernels read or write past an allocation. These checks run
on the host: every case here raises ValueError before a library call (CPU tensors throughout; the device check
comes after the size checks, so correctly sized CPU tensors fail on the device alone).
"""
import pytest

torch = pytest.importorskip("torch")

kvq = pytest.importorskip("decode_attention_quant_amd")

B, HKV, HQ, T = 2, 2, 8, 64


def _cache():
    c = kvq.KVCache(kvq.Shape(B, HKV, HQ, max_tokens=256), device="cpu")
    c.c.n_resid = 5   # host fields of a non-empty cache: the workspace size is then positive
    return c


def _kv(b=B, h=HKV, t=T, dtype=torch.float16):
    return torch.zeros((b, h, t, 128), dtype=dtype)


@pytest.mark.parametrize("k_shape", [(B - 1, HKV), (B, HKV + 1), (B + 1, HKV - 1)])
def test_append_rejects_leading_sizes(k_shape):
    c = _cache()
    with pytest.raises(ValueError, match="leading sizes"):
        kvq.kv_append_and_flush(c, _kv(*k_shape), _kv(*k_shape))
    assert (c.n_quant, c.n_resid) == (0, 5)


def test_append_rejects_dtype_and_device():
    c = _cache()
    with pytest.raises(ValueError, match="float16"):
        kvq.kv_append_and_flush(c, _kv(dtype=torch.float32), _kv(dtype=torch.float32))
    with pytest.raises(ValueError, match="CUDA tensor"):
        kvq.kv_append_and_flush(c, _kv(), _kv())


def test_quant_rejects_sizes_of_inputs_and_tiles():
    shape = kvq.Shape(B, HKV, HQ, max_tokens=256)
    tiles = torch.zeros((B, HKV, 256 // 32, kvq.RECORD_BYTES), dtype=torch.uint8)
    with pytest.raises(ValueError, match="leading sizes"):
        kvq.kv_quant_keys_per_channel(shape, _kv(b=1), 0, tiles)
    with pytest.raises(ValueError, match="tiles holds"):
        kvq.kv_quant_values_per_token(shape, _kv(), 0, tiles[:1])
    with pytest.raises(ValueError, match="uint8"):
        kvq.kv_quant_keys_per_channel(shape, _kv(), 0, tiles.view(torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        kvq.kv_quant_keys_per_channel(shape, _kv(), 0, tiles.transpose(0, 1))
    with pytest.raises(ValueError, match="CUDA tensor"):
        kvq.kv_quant_keys_per_channel(shape, _kv(), 0, tiles)


def test_decode_rejects_query_output_and_workspace():
    c = _cache()
    need = kvq.kv_decode_attention_workspace_bytes(c)
    assert need > 0
    q = torch.zeros((B, HQ, 128), dtype=torch.float16)
    out = torch.zeros((B, HQ, 128), dtype=torch.float32)
    ws = torch.zeros(need, dtype=torch.uint8)
    with pytest.raises(ValueError, match="q must be"):
        kvq.kv_decode_attention(c, q[:1], out=out, workspace=ws)
    with pytest.raises(ValueError, match="q must be"):
        kvq.kv_decode_attention(c, q.float(), out=out, workspace=ws)
    with pytest.raises(ValueError, match="out must be"):
        kvq.kv_decode_attention(c, q, out=out.half(), workspace=ws)
    with pytest.raises(ValueError, match="out must be"):
        kvq.kv_decode_attention(c, q, out=out[:1], workspace=ws)
    with pytest.raises(ValueError, match="out must be"):
        kvq.kv_decode_attention(c, q, out=out.transpose(1, 2).contiguous().transpose(1, 2), workspace=ws)
    with pytest.raises(ValueError, match="workspace holds"):
        kvq.kv_decode_attention(c, q, out=out, workspace=ws[:need - 16])
    with pytest.raises(ValueError, match="CUDA tensor"):
        kvq.kv_decode_attention(c, q, out=out, workspace=ws)


def test_ragged_calls_reject_sizes():
    c = kvq.RaggedCache(kvq.Shape(B, HKV, HQ, max_tokens=256), device="cpu")
    k = torch.zeros((HKV, 40, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="KV heads"):
        kvq.kv_ragged_prefill(c, 0, k[:1], k[:1])
    with pytest.raises(ValueError, match="sequence index"):
        kvq.kv_ragged_prefill(c, B, k, k)
    with pytest.raises(ValueError, match="CUDA tensor"):
        kvq.kv_ragged_prefill(c, 0, k, k)
    tok = torch.zeros((B, HKV, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="leading sizes"):
        kvq.kv_ragged_append(c, tok[:1], tok[:1])
    with pytest.raises(ValueError, match="CUDA tensor"):
        kvq.kv_ragged_append(c, tok, tok)
    need = kvq.kv_ragged_workspace_bytes(c)
    q = torch.zeros((B, HQ, 128), dtype=torch.float16)
    out = torch.zeros((B, HQ, 128), dtype=torch.float32)
    ws = torch.zeros(need, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace holds"):
        kvq.kv_ragged_decode_attention(c, q, out=out, workspace=ws[:need // 2])
    with pytest.raises(ValueError, match="out must be"):
        kvq.kv_ragged_decode_step(c, tok, tok, q, out=out[:, :1], workspace=ws)
    with pytest.raises(ValueError, match="leading sizes"):
        kvq.kv_ragged_decode_step(c, tok[:, :1], tok[:, :1], q, out=out, workspace=ws)
    with pytest.raises(ValueError, match="CUDA tensor"):
        kvq.kv_ragged_decode_step(c, tok, tok, q, out=out, workspace=ws)
