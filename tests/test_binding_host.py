"""Host-side checks of the Python binding (no GPU): tensors are checked for type, dtype,
contiguity, size and GPU residence before any pointer crosses the C ABI, so a buffer that a
kernel would read or write past its end raises instead of reaching the device."""
import pytest
import torch

from sparse_kv_attention_dense_amd import binding as B


def test_buf_accepts_optional_none_and_rejects_missing():
    B._buf(None, "lse", B._F32, 8, optional=True)
    with pytest.raises(ValueError, match="required"):
        B._buf(None, "out", B._F32, 8)


def test_buf_rejects_non_tensors_and_wrong_dtype():
    with pytest.raises(TypeError, match="torch.Tensor"):
        B._buf([1, 2, 3], "idx", B._I32)
    with pytest.raises(TypeError, match="dtype"):
        B._buf(torch.zeros(64, dtype=torch.int64), "idx", B._I32, 64)


def test_buf_rejects_strided_views_and_short_buffers():
    t = torch.zeros((8, 16), dtype=torch.float32)
    with pytest.raises(ValueError, match="contiguous"):
        B._buf(t.t(), "logits", B._F32, 128)
    with pytest.raises(ValueError, match="needs 129"):
        B._buf(t, "logits", B._F32, 129)


def test_buf_rejects_host_memory_last():
    # every other property right: only the device is wrong
    with pytest.raises(ValueError, match="GPU memory"):
        B._buf(torch.zeros(128, dtype=torch.float32), "out", B._F32, 128)


def _kv(dtype=torch.bfloat16, shape=(2, 2, 64, 128)):
    return torch.zeros(shape, dtype=dtype), torch.zeros(shape, dtype=dtype)


def test_kvdesc_rejects_bad_cache_tensors():
    lens = torch.zeros(2, dtype=torch.int32)
    k, v = _kv(torch.float16)
    with pytest.raises(TypeError, match="float32 or torch.bfloat16"):
        B.KVDesc(k, v, lens, 64, 8)
    k, v = _kv()
    with pytest.raises(TypeError, match="lens"):
        B.KVDesc(k, v, lens.long(), 64, 8)
    with pytest.raises(ValueError, match="contiguous"):
        B.KVDesc(k.transpose(2, 3), v.transpose(2, 3), lens, 64, 8)
    with pytest.raises(ValueError, match="differs"):
        B.KVDesc(k, v[:, :, :32].contiguous(), lens, 64, 8)
    with pytest.raises(ValueError, match="sequences"):
        B.KVDesc(k[:1].contiguous(), v[:1].contiguous(), lens, 64, 8)
    with pytest.raises(ValueError, match="expected"):
        B.KVDesc(k[0], v[0], lens, 64, 8)


def test_kvdesc_rejects_inconsistent_pages():
    lens = torch.zeros(2, dtype=torch.int32)
    k, v = _kv(shape=(10, 2, 16, 128))
    bt = torch.zeros((2, 5), dtype=torch.int32)
    with pytest.raises(ValueError, match="block_size"):
        B.KVDesc(k, v, lens, 64, 8, block_table=bt, block_size=32)
    with pytest.raises(TypeError, match="block_table"):
        B.KVDesc(k, v, lens, 64, 8, block_table=bt.long(), block_size=16)


def test_kvdesc_needs_gpu_memory():
    k, v = _kv()
    with pytest.raises(ValueError, match="GPU memory"):
        B.KVDesc(k, v, torch.zeros(2, dtype=torch.int32), 64, 8)
