"""Host-side checks of the C ABI (no GPU): the library loads, exports every symbol the header
declares, and rejects bad arguments before enqueuing anything (fake device pointers are never
dereferenced on these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qjl.h")

qjl = pytest.importorskip("bit_kv_cache_qjl_amd")

FAKE = 0x7F0000001000          # 16-byte aligned, never dereferenced
MIS = FAKE + 8                 # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qjl_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"qjl_quantize_keys", "qjl_quantize_values", "qjl_decode_attention"} <= set(names)
    for n in names:
        assert hasattr(qjl.lib, n), n
        assert ctypes.cast(getattr(qjl.lib, n), ctypes.c_void_p).value


def test_status_strings():
    assert qjl.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert qjl.status_string(s) not in ("ok", "unknown status")
    assert qjl.status_string(17) == "unknown status"


def keys_call(**kw):
    a = dict(K=FAKE, kdt=0, B=1, T=64, Hkv=2, d=128, sK_b=64 * 2 * 128, sK_t=2 * 128, sK_h=128, S_in=FAKE, m=256,
             S_out=FAKE, m_out=256, oidx=FAKE, n_out=4, bits=FAKE, norms=FAKE, Ncap=64, t0=0, stream=0)
    a.update(kw)
    return qjl.lib.qjl_quantize_keys(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(kdt=5), qjl.QJL_ERR_INVALID_ARG),
    (dict(d=64), qjl.QJL_ERR_UNSUPPORTED),
    (dict(m=48), qjl.QJL_ERR_UNSUPPORTED),
    (dict(m=768, m_out=512), qjl.QJL_ERR_UNSUPPORTED),
    (dict(n_out=17), qjl.QJL_ERR_UNSUPPORTED),
    (dict(m_out=0, n_out=4), qjl.QJL_ERR_INVALID_ARG),
    (dict(T=65, Ncap=64), qjl.QJL_ERR_INVALID_ARG),
    (dict(t0=10), qjl.QJL_ERR_INVALID_ARG),
    (dict(K=0), qjl.QJL_ERR_INVALID_ARG),
    (dict(oidx=0), qjl.QJL_ERR_INVALID_ARG),
    (dict(K=MIS), qjl.QJL_ERR_MISALIGNED),
    (dict(bits=MIS), qjl.QJL_ERR_MISALIGNED),
    (dict(sK_t=2 * 128 + 4), qjl.QJL_ERR_MISALIGNED),
    (dict(Hkv=0), qjl.QJL_ERR_INVALID_ARG),
])
def test_quantize_keys_rejects(kw, status):
    assert keys_call(**kw) == status
    assert qjl.last_error() != ""


def test_quantize_keys_empty_is_noop():
    assert keys_call(T=0, K=0) == qjl.QJL_OK
    assert keys_call(B=0, K=0) == qjl.QJL_OK
    assert qjl.last_error() == ""


def values_call(**kw):
    a = dict(V=FAKE, vdt=0, B=1, T=64, Hkv=2, d=128, sV_b=64 * 2 * 128, sV_t=2 * 128, sV_h=128, nbits=2, codes=FAKE,
             meta=FAKE, Ncap=64, t0=0, stream=0)
    a.update(kw)
    return qjl.lib.qjl_quantize_values(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(nbits=1), qjl.QJL_ERR_UNSUPPORTED),
    (dict(nbits=8), qjl.QJL_ERR_UNSUPPORTED),
    (dict(d=256), qjl.QJL_ERR_UNSUPPORTED),
    (dict(codes=0), qjl.QJL_ERR_INVALID_ARG),
    (dict(meta=MIS), qjl.QJL_ERR_MISALIGNED),
    (dict(vdt=1, sV_h=130), qjl.QJL_ERR_MISALIGNED),
    (dict(T=100), qjl.QJL_ERR_INVALID_ARG),
])
def test_quantize_values_rejects(kw, status):
    assert values_call(**kw) == status


def test_quantize_values_empty_is_noop():
    assert values_call(T=0, V=0) == qjl.QJL_OK
    assert values_call(B=0, V=0) == qjl.QJL_OK


def decode_call(ws_bytes=None, **kw):
    a = dict(Q=FAKE, qdt=0, B=2, Hq=8, Hkv=2, d=128, N=1000, S_in=FAKE, m=256, S_out=FAKE, m_out=256, oidx=FAKE,
             n_out=3, bits=FAKE, norms=FAKE, Ncap=1024, vmode=0, codes=FAKE, meta=FAKE, V_f32=0, nbits=2,
             sm_scale=0.0, estimator=0, path=0, out=FAKE, scores=0, nsplit=0, ws=FAKE, ws_bytes=0, stream=0)
    a.update(kw)
    if ws_bytes is None:
        a["ws_bytes"] = qjl.lib.qjl_decode_workspace_size(a["B"], a["Hq"], a["Hkv"], 128, a["N"], a["m"], a["m_out"],
                                                          a["nsplit"]) - 4
    else:
        a["ws_bytes"] = ws_bytes
    return qjl.lib.qjl_decode_attention(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=9), qjl.QJL_ERR_INVALID_ARG),
    (dict(N=2000), qjl.QJL_ERR_INVALID_ARG),
    (dict(m=384, m_out=384), qjl.QJL_ERR_UNSUPPORTED),
    (dict(m=256, m_out=128), qjl.QJL_ERR_UNSUPPORTED),
    (dict(nbits=5), qjl.QJL_ERR_UNSUPPORTED),
    (dict(nbits=4, m=512, m_out=512), qjl.QJL_ERR_UNSUPPORTED),   # 3- and 4-bit codes: matrix-core shapes only
    (dict(nbits=3, m=512, m_out=512), qjl.QJL_ERR_UNSUPPORTED),
    (dict(vmode=1), qjl.QJL_ERR_INVALID_ARG),          # fp32 values but V_f32 is null
    (dict(vmode=7), qjl.QJL_ERR_INVALID_ARG),
    (dict(estimator=2), qjl.QJL_ERR_INVALID_ARG),
    (dict(estimator=-1), qjl.QJL_ERR_INVALID_ARG),
    (dict(path=3), qjl.QJL_ERR_INVALID_ARG),
    (dict(path=-1), qjl.QJL_ERR_INVALID_ARG),
    (dict(path=1, m=512, m_out=512), qjl.QJL_ERR_UNSUPPORTED),     # matrix cores: sketches up to 512 bits
    (dict(path=1, vmode=1, V_f32=FAKE), qjl.QJL_ERR_UNSUPPORTED),  # matrix cores: value codes only
    (dict(path=2, nbits=3), qjl.QJL_ERR_UNSUPPORTED),              # vector units: 2-bit codes only
    (dict(path=2, nbits=4), qjl.QJL_ERR_UNSUPPORTED),
    (dict(out=MIS), qjl.QJL_ERR_MISALIGNED),
    (dict(scores=MIS), qjl.QJL_ERR_MISALIGNED),
    (dict(nsplit=5000, ws_bytes=1 << 30), qjl.QJL_ERR_UNSUPPORTED),
    (dict(), qjl.QJL_ERR_WORKSPACE),                    # 4 bytes short
    (dict(path=1), qjl.QJL_ERR_WORKSPACE),              # a valid path: the next check fails
    (dict(path=2), qjl.QJL_ERR_WORKSPACE),
    (dict(ws=0), qjl.QJL_ERR_WORKSPACE),
])
def test_decode_rejects(kw, status):
    assert decode_call(**kw) == status


def test_decode_workspace_size_formula():
    B, Hq, Hkv, N, m, m_out = 8, 32, 32, 32768, 256, 256
    for nsplit in (1, 4, 7):
        ws = qjl.decode_workspace_size(B, Hq, Hkv, N, m, m_out, nsplit)
        sq = B * Hq * (m + m_out) * 4
        qconst = B * Hq * 4 * 4
        part = B * Hq * nsplit * 130 * 4
        r = lambda x: (x + 255) // 256 * 256
        assert ws == r(sq) + r(qconst) + r(part)
    assert qjl.decode_workspace_size(B, Hq, Hkv, N, m, m_out, 0) >= qjl.decode_workspace_size(B, Hq, Hkv, N, m, m_out, 1)
    assert qjl.decode_workspace_size(B, 9, 2, N, m, m_out) == 0


def test_timer_api():
    qjl.timer_enable(True)
    assert qjl.timer_read("decode") == (0, 0.0)
    qjl.timer_enable(False)
    with pytest.raises(qjl.QJLError):
        qjl.timer_read("nope")


def step_call(ws_bytes=None, **kw):
    a = dict(Q=FAKE, K_new=FAKE, V_new=FAKE, dt=0, B=2, Hq=8, Hkv=2, d=128, N=1000, sK_b=2 * 128, sK_h=128,
             sV_b=2 * 128, sV_h=128, S_in=FAKE, m=256, S_out=FAKE, m_out=256, oidx=FAKE, n_out=3, bits=FAKE,
             norms=FAKE, codes=FAKE, meta=FAKE, Ncap=1024, nbits=2, sm_scale=0.0, estimator=0, path=0, out=FAKE, scores=0,
             nsplit=0, ws=FAKE, ws_bytes=0, stream=0)
    a.update(kw)
    if ws_bytes is None:
        a["ws_bytes"] = qjl.lib.qjl_decode_workspace_size(a["B"], a["Hq"], a["Hkv"], 128, a["N"], a["m"], a["m_out"],
                                                          a["nsplit"]) - 4
    else:
        a["ws_bytes"] = ws_bytes
    return qjl.lib.qjl_decode_step(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), qjl.QJL_ERR_INVALID_ARG),               # no position for the new token
    (dict(N=1025), qjl.QJL_ERR_INVALID_ARG),
    (dict(dt=3), qjl.QJL_ERR_INVALID_ARG),
    (dict(Hq=9), qjl.QJL_ERR_INVALID_ARG),
    (dict(estimator=5), qjl.QJL_ERR_INVALID_ARG),
    (dict(nbits=5), qjl.QJL_ERR_UNSUPPORTED),
    (dict(m=256, m_out=128), qjl.QJL_ERR_UNSUPPORTED),
    (dict(K_new=0), qjl.QJL_ERR_INVALID_ARG),
    (dict(codes=0), qjl.QJL_ERR_INVALID_ARG),
    (dict(sK_h=-128), qjl.QJL_ERR_INVALID_ARG),
    (dict(sV_h=130), qjl.QJL_ERR_MISALIGNED),
    (dict(dt=1, sK_b=2 * 128 + 2), qjl.QJL_ERR_MISALIGNED),
    (dict(meta=MIS), qjl.QJL_ERR_MISALIGNED),
    (dict(nsplit=5000, ws_bytes=1 << 30), qjl.QJL_ERR_UNSUPPORTED),
    (dict(), qjl.QJL_ERR_WORKSPACE),                    # 4 bytes short
    (dict(ws=0), qjl.QJL_ERR_WORKSPACE),
])
def test_decode_step_rejects(kw, status):
    assert step_call(**kw) == status
    assert qjl.last_error() != ""


def test_decode_step_empty_batch_is_noop():
    assert step_call(B=0, ws=0, ws_bytes=0) == qjl.QJL_OK


def select_call(ws_bytes=None, **kw):
    a = dict(K=FAKE, kdt=0, B=2, T=100, Hkv=4, d=128, sK_b=100 * 4 * 128, sK_t=4 * 128, sK_h=128, n_out=4,
             oidx=FAKE, ws=FAKE, ws_bytes=0, stream=0)
    a.update(kw)
    a["ws_bytes"] = (qjl.lib.qjl_select_outliers_workspace_size(a["B"], a["T"], a["Hkv"], 128) - 8
                     if ws_bytes is None else ws_bytes)
    return qjl.lib.qjl_select_outliers(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(kdt=2), qjl.QJL_ERR_INVALID_ARG),
    (dict(T=-1), qjl.QJL_ERR_INVALID_ARG),
    (dict(n_out=17), qjl.QJL_ERR_UNSUPPORTED),
    (dict(d=64), qjl.QJL_ERR_UNSUPPORTED),
    (dict(oidx=0), qjl.QJL_ERR_INVALID_ARG),
    (dict(K=0), qjl.QJL_ERR_INVALID_ARG),
    (dict(sK_t=4 * 128 + 4), qjl.QJL_ERR_MISALIGNED),
    (dict(oidx=MIS), qjl.QJL_ERR_MISALIGNED),
    (dict(), qjl.QJL_ERR_WORKSPACE),                    # 8 bytes short
    (dict(ws=0), qjl.QJL_ERR_WORKSPACE),
])
def test_select_outliers_rejects(kw, status):
    assert select_call(**kw) == status
    assert qjl.last_error() != ""


def test_select_outliers_no_channels_is_noop():
    assert select_call(n_out=0, K=0, oidx=0, ws=0) == qjl.QJL_OK


def test_select_outliers_workspace_formula():
    # ~1024 workgroups of >= 256 tokens over (sequence, head): one fp64 sum per channel each
    assert qjl.lib.qjl_select_outliers_workspace_size(1, 65536, 8, 128) == 128 * 8 * 128 * 8
    assert qjl.lib.qjl_select_outliers_workspace_size(2, 100, 4, 128) == ((1 * 2 * 4 * 128 * 8 + 255) // 256) * 256
    assert qjl.lib.qjl_select_outliers_workspace_size(1, 10, 4, 64) == 0


def step_no_alloc_call(**kw):
    a = dict(Q=FAKE, K_new=FAKE, V_new=FAKE, dt=0, B=2, Hq=8, Hkv=2, d=128, N=1000, sK_b=2 * 128, sK_h=128,
             sV_b=2 * 128, sV_h=128, S_in=FAKE, m=256, S_out=FAKE, m_out=256, oidx=FAKE, n_out=3, bits=FAKE,
             norms=FAKE, codes=FAKE, meta=FAKE, Ncap=1024, nbits=2, sm_scale=0.0, estimator=0, path=0, out=FAKE, scores=0,
             nsplit=0, stream=0)
    a.update(kw)
    return qjl.lib.qjl_decode_step_no_alloc(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), qjl.QJL_ERR_INVALID_ARG),
    (dict(N=1025), qjl.QJL_ERR_INVALID_ARG),
    (dict(Hq=9), qjl.QJL_ERR_INVALID_ARG),
    (dict(nbits=5), qjl.QJL_ERR_UNSUPPORTED),
    (dict(K_new=0), qjl.QJL_ERR_INVALID_ARG),
    (dict(meta=MIS), qjl.QJL_ERR_MISALIGNED),
    # 64 x 128 query heads: the query operands alone need 16 MiB, beyond the fixed 8 MiB scratch
    (dict(B=64, Hq=128, Hkv=8), qjl.QJL_ERR_WORKSPACE),
])
def test_decode_step_no_alloc_rejects_before_touching_a_device(kw, status):
    """Every argument error, and a workspace need beyond the fixed scratch, is reported before the
    entry point looks for the device scratch (so no GPU is needed to see them)."""
    assert step_no_alloc_call(**kw) == status
    assert qjl.last_error() != ""
    if status == qjl.QJL_ERR_WORKSPACE:
        assert "fixed scratch" in qjl.last_error()
        assert qjl.lib.qjl_decode_workspace_size(64, 128, 8, 128, 1000, 256, 256, 0) > qjl.NO_ALLOC_SCRATCH_BYTES


def test_decode_step_no_alloc_empty_batch_is_noop():
    assert step_no_alloc_call(B=0) == qjl.QJL_OK


def test_no_alloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define QJL_NO_ALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == qjl.NO_ALLOC_SCRATCH_BYTES
