"""GPU parity of outlier-channel selection (qjl_select_outliers) with the oracle: the chosen channel
sets must be identical (an index result: bit-exact).  Both sides sum bf16 magnitudes in fp64, where
the sums of these inputs are exact, so equal means are equal on both sides and the tie order (lower
channel first) decides the same way."""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qjl = pytest.importorskip("bit_kv_cache_qjl_amd")

W = si.WORKLOADS
CASES = {
    "llama2_mha": W["llama2_7b_decode"].scaled(B=2, Hq=3, Hkv=3, N=1500),
    "llama3_gqa": W["llama3_8b_gqa_decode"].scaled(B=2, Hq=8, Hkv=2, N=1100),
    "llama31_70b_gqa": W["llama31_70b_gqa_decode"].scaled(B=1, Hq=16, Hkv=2, N=777),
    "prefill_64k_heads": W["prefill_quantize_64k"].scaled(N=3000),
    "fp32_keys": W["llama3_8b_gqa_decode"].scaled(B=2, Hq=4, Hkv=4, N=513, dtype="f32"),
}


def gpu_select(K_dev, n_out):
    out = qjl.select_outliers(K_dev, n_out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_select_outliers_parity(name):
    w = CASES[name]
    log(f"[select_outliers] {name} B={w.B} T={w.N} Hkv={w.Hkv} n_out={w.n_out} {w.dtype}")
    planted = si.outlier_channels(w)
    K = si.keys(w, planted)
    got = gpu_select(to_dev(K, w.dtype), w.n_out)
    ref = oracle.select_outliers(K, w.n_out)
    np.testing.assert_array_equal(got, ref)
    # the generator scales its outlier channels by 20-50x: the selection must find exactly those
    np.testing.assert_array_equal(got, np.sort(planted, axis=1))


@pytest.mark.parametrize("n_out", [1, 7, 16])
def test_select_outliers_counts_and_strides(n_out):
    """Every n_out on plain Gaussian keys (no planted channels: the ranking is decided by small
    differences of the means), on a token-strided view of a larger tensor."""
    rng = np.random.default_rng(100 + n_out)
    big = si.round_bf16(rng.standard_normal((3, 2 * 700, 5, 128)).astype(np.float32))
    K = big[:, ::2]
    dev = to_dev(big, "bf16")[:, ::2]
    assert not dev.is_contiguous()
    np.testing.assert_array_equal(gpu_select(dev, n_out), oracle.select_outliers(K, n_out))


def test_select_outliers_exact_ties():
    """Integer-valued keys whose channel sums tie exactly: the lower channel must win on both sides."""
    B, T, Hkv = 2, 300, 3
    K = np.ones((B, T, Hkv, 128), dtype=np.float32)
    K[:, :, 0, [5, 9, 77]] = 3.0                 # three equal winners
    K[:, :, 1, [100, 3]] = -2.0                  # two equal winners, signs do not matter
    K[0, :, 1, 50] = 4.0                         # mean 2.0 over both sequences: ties with 100 and 3
    K[1, :, 1, 50] = 0.0
    K[:, :, 2, :] = 0.0                          # all zero: channels 0.. in order
    got = gpu_select(to_dev(K, "bf16"), 4)
    ref = oracle.select_outliers(K, 4)
    np.testing.assert_array_equal(got, ref)
    assert got[0].tolist() == [0, 5, 9, 77] and got[1].tolist() == [0, 3, 50, 100] and got[2].tolist() == [0, 1, 2, 3]


def test_select_outliers_empty_batch_and_determinism():
    empty = torch.empty((0, 10, 2, 128), dtype=torch.bfloat16, device="cuda")
    assert gpu_select(empty, 3).tolist() == oracle.select_outliers(np.zeros((0, 10, 2, 128)), 3).tolist() == [[0, 1, 2]] * 2
    w = CASES["llama3_gqa"]
    K = to_dev(si.keys(w, si.outlier_channels(w)), w.dtype)
    a, b = gpu_select(K, 5), gpu_select(K, 5)
    np.testing.assert_array_equal(a, b)


def test_select_outliers_full_prefill_shape():
    """65536 tokens x 8 KV heads (the prefill quantize workload), against the oracle."""
    w = W["prefill_quantize_64k"]
    planted = si.outlier_channels(w)
    K = si.keys(w, planted)
    log(f"[select_outliers] full {w.name}: B={w.B} T={w.N} Hkv={w.Hkv}")
    got = gpu_select(to_dev(K, w.dtype), w.n_out)
    np.testing.assert_array_equal(got, oracle.select_outliers(K, w.n_out))
    np.testing.assert_array_equal(got, np.sort(planted, axis=1))
