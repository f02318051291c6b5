"""Host-side checks of the Python binding's argument validation (no GPU): mistakes that the C ABI
cannot see from raw pointers (an int64 outlier list read as int32, JL matrices of another dtype than the
keys, a cache of the wrong shape, code tiles of another width) are refused before any call."""
import pytest

torch = pytest.importorskip("torch")
qjl = pytest.importorskip("bit_kv_cache_qjl_amd")


def test_sketch_args_accepts_matching_dtypes_and_counts():
    S_in = torch.zeros((256, 128), dtype=torch.bfloat16)
    S_out = torch.zeros((256, 128), dtype=torch.bfloat16)
    oidx = torch.zeros((8, 5), dtype=torch.int32)
    assert qjl._sketch_args(S_in, S_out, oidx, torch.bfloat16, 8, 128) == (256, 256, 5)
    assert qjl._sketch_args(S_in, None, None, torch.bfloat16, 8, 128) == (256, 0, 0)


@pytest.mark.parametrize("what,exc", [
    ("int64_outliers", TypeError),
    ("outliers_wrong_heads", ValueError),
    ("s_in_f32_for_bf16_keys", TypeError),
    ("s_out_other_dtype", TypeError),
    ("s_in_wrong_width", ValueError),
])
def test_sketch_args_refuses(what, exc):
    S_in = torch.zeros((256, 128), dtype=torch.bfloat16)
    S_out = torch.zeros((256, 128), dtype=torch.bfloat16)
    oidx = torch.zeros((8, 5), dtype=torch.int32)
    if what == "int64_outliers":
        oidx = oidx.long()
    elif what == "outliers_wrong_heads":
        oidx = torch.zeros((4, 5), dtype=torch.int32)
    elif what == "s_in_f32_for_bf16_keys":
        S_in = S_in.float()
    elif what == "s_out_other_dtype":
        S_out = S_out.float()
    elif what == "s_in_wrong_width":
        S_in = torch.zeros((256, 64), dtype=torch.bfloat16)
    with pytest.raises(exc):
        qjl._sketch_args(S_in, S_out, oidx, torch.bfloat16, 8, 128)


def test_key_cache_args():
    bits = torch.zeros((4, 8, 100, 16), dtype=torch.int32)
    norms = torch.zeros((4, 8, 100, 2), dtype=torch.float16)
    assert qjl._key_cache_args(bits, norms, 4, 8, 256, 256) == 100
    assert qjl._key_cache_args(bits, norms, 2, 8, 256, 256) == 100          # a prefix of the sequences
    with pytest.raises(ValueError):
        qjl._key_cache_args(bits, norms, 5, 8, 256, 256)                   # more sequences than the cache
    with pytest.raises(ValueError):
        qjl._key_cache_args(bits, norms, 4, 4, 256, 256)                   # other KV-head count
    with pytest.raises(ValueError):
        qjl._key_cache_args(bits, norms, 4, 8, 256, 0)                     # other sketch width
    with pytest.raises(ValueError):
        qjl._key_cache_args(bits, norms[:, :, :99], 4, 8, 256, 256)        # norms of another capacity
    with pytest.raises(TypeError):
        qjl._key_cache_args(bits, norms.float(), 4, 8, 256, 256)


def test_value_cache_args():
    for nbits in (2, 3, 4):
        codes = torch.zeros((2, 8, 4, 128, nbits), dtype=torch.int32)
        meta = torch.zeros((2, 8, 100, 2), dtype=torch.float16)
        assert qjl._value_cache_args(codes, meta, 2, 8, nbits, 128) == 100
        assert qjl._value_cache_args(codes, meta, 2, 8, nbits, 128, 100) == 100
        with pytest.raises(ValueError):
            qjl._value_cache_args(codes, meta, 2, 8, 6 - nbits if nbits != 3 else 2, 128)   # tiles of another width
        with pytest.raises(ValueError):
            qjl._value_cache_args(codes, meta, 2, 8, nbits, 128, 101)                    # key cache of another capacity
        with pytest.raises(ValueError):
            qjl._value_cache_args(codes[:, :, :3], meta, 2, 8, nbits, 128)              # too few tiles
        with pytest.raises(ValueError):
            qjl._value_cache_args(codes, meta, 3, 8, nbits, 128)
    with pytest.raises(ValueError):
        qjl._value_cache_args(codes, meta, 2, 8, 5, 128)


def test_host_tensors_are_refused():
    K = torch.zeros((1, 4, 2, 128), dtype=torch.bfloat16)
    S = torch.zeros((256, 128), dtype=torch.bfloat16)
    bits = torch.zeros((1, 2, 4, 8), dtype=torch.int32)
    norms = torch.zeros((1, 2, 4, 2), dtype=torch.float16)
    with pytest.raises(ValueError, match="device"):
        qjl.quantize_keys(K, S, None, None, bits, norms)
