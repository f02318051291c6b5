"""HIP-graph capture of the decode entry points: a step captured once and replayed several times, with
other eager work on the same stream in between, gives bit-for-bit the eager result on every replay.
(The library launches kernels only: no allocation, no memset, no synchronization inside a call.)"""
import numpy as np
import pytest

import oracle
import seeded_inputs as si
from gpu_util import bits_dev, code_tiles_of_rows, inputs, log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
qjl = pytest.importorskip("bit_kv_cache_qjl_amd")

W = si.WORKLOADS
CASES = {
    "llama3_gqa": W["llama3_8b_gqa_decode"].scaled(B=2, Hq=8, Hkv=2, N=1100),
    "llama31_70b_gqa_4bit": W["llama31_70b_gqa_decode"].scaled(B=1, Hq=16, Hkv=2, N=777, nbits=4),
}


def device_cache(w, x, Ncap):
    kq = oracle.quantize_keys(x["K"], x["S_in"], x["S_out"], x["oidx"])
    vq = oracle.quantize_values(x["V"], w.nbits)
    bits = np.zeros((w.B, w.Hkv, Ncap, (w.m + w.m_out) // 32), np.uint32)
    bits[:, :, :w.N] = kq["bits"]
    norms = np.zeros((w.B, w.Hkv, Ncap, 2), np.float16)
    norms[:, :, :w.N] = kq["norms"]
    meta = np.zeros((w.B, w.Hkv, Ncap, 2), np.float16)
    meta[:, :, :w.N] = vq["meta"]
    tiles = code_tiles_of_rows(vq["codes"], w.nbits, Ncap, w.d)
    return qjl.Cache(bits=bits_dev(bits, w.m, w.m_out), norms=torch.from_numpy(norms).cuda(),
                     codes=torch.from_numpy(tiles.view(np.int32)).cuda(), meta=torch.from_numpy(meta).cuda(),
                     m=w.m, m_out=w.m_out, nbits=w.nbits)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_graph_replays_match_eager(name):
    w = CASES[name]
    N, Ncap = w.N, w.N + 3
    log(f"[graph] decode_step {name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={N} nbits={w.nbits}")
    x = inputs(w)
    Q = to_dev(x["Q"], w.dtype)
    Kd, Vd = to_dev(x["K"], w.dtype), to_dev(x["V"], w.dtype)
    S_in, S_out = to_dev(x["S_in"], w.dtype), to_dev(x["S_out"], w.dtype)
    oidx = torch.from_numpy(x["oidx"]).cuda()
    cache = device_cache(w, x, Ncap)
    ws = torch.empty(qjl.decode_workspace_size(w.B, w.Hq, w.Hkv, N, w.m, w.m_out, 0), dtype=torch.uint8, device="cuda")
    k_new, v_new = Kd[:, N - 1:N].clone(), Vd[:, N - 1:N].clone()

    out_eager = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    qjl.decode_step(Q, k_new, v_new, S_in, S_out, oidx, cache, N, out_eager, workspace=ws)
    torch.cuda.synchronize()
    ref = out_eager.clone()
    cache_ref = {f: getattr(cache, f).clone() for f in ("bits", "norms", "codes", "meta")}

    out = torch.full_like(out_eager, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            qjl.decode_step(Q, k_new, v_new, S_in, S_out, oidx, cache, N, out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other = torch.empty_like(out_eager)
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs from the eager step"
        for f, t in cache_ref.items():
            assert torch.equal(getattr(cache, f), t), f"replay {r} changed the cache ({f})"
        # eager work on the same buffers and workspace between replays
        qjl.decode_step(Q, k_new, v_new, S_in, S_out, oidx, cache, N, other, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(other, ref)


def test_decode_attention_graph_with_split_merge():
    """A forced split (several chunks per KV head, so the merge launch is part of the graph)."""
    w = CASES["llama3_gqa"]
    N = w.N
    log(f"[graph] decode_attention split N={N}")
    x = inputs(w)
    Q = to_dev(x["Q"], w.dtype)
    S_in, S_out = to_dev(x["S_in"], w.dtype), to_dev(x["S_out"], w.dtype)
    oidx = torch.from_numpy(x["oidx"]).cuda()
    cache = device_cache(w, x, N)
    ws = torch.empty(qjl.decode_workspace_size(w.B, w.Hq, w.Hkv, N, w.m, w.m_out, 5), dtype=torch.uint8, device="cuda")
    kw = dict(codes=cache.codes, meta=cache.meta, nbits=w.nbits, nsplit=5, workspace=ws)
    ref = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    qjl.decode_attention(Q, S_in, S_out, oidx, cache.bits, cache.norms, N, ref, **kw)
    torch.cuda.synchronize()
    out = torch.full_like(ref, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            qjl.decode_attention(Q, S_in, S_out, oidx, cache.bits, cache.norms, N, out, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs"
        qjl.decode_attention(Q, S_in, S_out, oidx, cache.bits, cache.norms, N // 2, torch.empty_like(ref), **kw)
        torch.cuda.synchronize()
