"""GPU check of qjl_decode_step_no_alloc (the decode step whose workspace is the library's fixed
device scratch array) against qjl_decode_step with a caller-allocated workspace, through the C ABI.

Two calls in a row, the second with a smaller input (fewer sequences, heads and positions, and a single
context chunk instead of two): the scratch keeps the first call's contents, and the second call must not
depend on them.  Each call runs both entry points on two copies of the same oracle-built cache prefix;
the appended rows and the outputs must be identical (the same kernels on the same inputs), and the
outputs must match the oracle on the cache the GPU wrote (2e-3 max-abs).
"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import bits_np, check_decode, code_rows_of_tiles, inputs, log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qjl = pytest.importorskip("bit_kv_cache_qjl_amd")
from bit_kv_cache_qjl_amd import layout  # noqa: E402

W70 = si.WORKLOADS["llama31_70b_gqa_decode"]
CALLS = [W70.scaled(B=2, Hq=16, Hkv=2, N=777), W70.scaled(B=1, Hq=8, Hkv=1, N=300)]


def prefix_cache(w, kq, vq, n_prefix: int):
    """Device cache of capacity N holding the oracle's rows 0 .. n_prefix-1 (zeros after)."""
    Wd = (w.m + w.m_out) // 32
    bits = np.zeros((w.B, w.Hkv, w.N, Wd), dtype=np.uint32)
    bits[:, :, :n_prefix] = kq["bits"][:, :, :n_prefix]
    norms = np.zeros((w.B, w.Hkv, w.N, 2), dtype=np.float16)
    norms[:, :, :n_prefix] = kq["norms"][:, :, :n_prefix]
    codes = np.zeros((w.B, w.Hkv, w.N, w.d), dtype=np.uint8)
    codes[:, :, :n_prefix] = oracle.unpack_codes(vq["codes"][:, :, :n_prefix], w.nbits, w.d)
    meta = np.zeros((w.B, w.Hkv, w.N, 2), dtype=np.float16)
    meta[:, :, :n_prefix] = vq["meta"][:, :, :n_prefix]
    return qjl.Cache(bits=torch.from_numpy(layout.bits_to_stored(bits, w.m, w.m_out).view(np.int32)).cuda(),
                     norms=torch.from_numpy(norms).cuda(),
                     codes=torch.from_numpy(layout.tiles_from_codes(codes, w.nbits, w.N).view(np.int32)).cuda(),
                     meta=torch.from_numpy(meta).cuda(), m=w.m, m_out=w.m_out, nbits=w.nbits)


def test_no_alloc_step_matches_workspace_step():
    for i, w in enumerate(CALLS):
        N = w.N
        need = qjl.decode_workspace_size(w.B, w.Hq, w.Hkv, N, w.m, w.m_out)
        assert 0 < need <= qjl.NO_ALLOC_SCRATCH_BYTES
        log(f"[no_alloc] call {i}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={N} (workspace {need} bytes)")
        x = inputs(w)
        kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
        vq = oracle.quantize_values(x["V"], w.nbits)
        Q = to_dev(x["Q"], w.dtype)
        Kd, Vd = to_dev(x["K"], w.dtype), to_dev(x["V"], w.dtype)
        S_in, S_out = to_dev(x["S_in"], w.dtype), to_dev(x["S_out"], w.dtype)
        od = torch.from_numpy(x["oidx"]).cuda()
        ca, cb = prefix_cache(w, kq, vq, N - 1), prefix_cache(w, kq, vq, N - 1)
        out_a = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
        out_b = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
        qjl.decode_step(Q, Kd[:, N - 1:N], Vd[:, N - 1:N], S_in, S_out, od, ca, N, out_a)
        qjl.decode_step_no_alloc(Q, Kd[:, N - 1:N], Vd[:, N - 1:N], S_in, S_out, od, cb, N, out_b)
        torch.cuda.synchronize()
        for f in ("bits", "norms", "codes", "meta"):
            assert torch.equal(getattr(ca, f), getattr(cb, f)), f"call {i}: cache {f} differs"
        assert torch.equal(out_a, out_b), f"call {i}: outputs differ"
        # the oracle on the cache the GPU wrote (identical inputs on both sides)
        cache_np = {"bits": bits_np(cb.bits, w.m, w.m_out), "norms": cb.norms.cpu().numpy(),
                    "codes": code_rows_of_tiles(cb.codes, w.nbits, N), "meta": cb.meta.cpu().numpy()}
        units = [(b, hq) for b in range(w.B) for hq in range(w.Hq)]
        check_decode(w, x["Q"], x["S_in"], x["S_out"], x["oidx"], cache_np, N, out_b.cpu().numpy(), None, units,
                     what=f"no_alloc call {i}")


def test_no_alloc_step_rejects_sizes_beyond_the_scratch():
    w = W70.scaled(B=64, Hq=128, Hkv=8, N=64)
    assert qjl.decode_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.m, w.m_out) > qjl.NO_ALLOC_SCRATCH_BYTES
    cache = qjl.alloc_cache(w.B, w.Hkv, w.N, w.m, w.m_out, w.nbits)
    Q = torch.zeros((w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    K1 = torch.zeros((w.B, 1, w.Hkv, w.d), dtype=torch.bfloat16, device="cuda")
    S = torch.zeros((w.m, w.d), dtype=torch.bfloat16, device="cuda")
    od = torch.zeros((w.Hkv, w.n_out), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    with pytest.raises(qjl.QJLError) as e:
        qjl.decode_step_no_alloc(Q, K1, K1, S, S, od, cache, w.N, out)
    assert e.value.status == qjl.QJL_ERR_WORKSPACE
    assert "fixed scratch" in qjl.last_error()
