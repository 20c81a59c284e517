"""C-ABI checks that need no GPU: exports, error codes, planning (CPU only).

Every call here either has an invalid argument or no work, so the library returns before any HIP
call; no kernel is launched.
"""

import ctypes
import math
import re
import subprocess

import pytest

import io_aware_tiled_amd as fa

OK, INVALID, UNSUPPORTED = fa.FATTN_OK, fa.FATTN_ERR_INVALID, fa.FATTN_ERR_UNSUPPORTED
BF16, F32 = fa.FATTN_BF16, fa.FATTN_F32
P = 0x10000  # a 16-byte aligned stand-in pointer; never dereferenced in these tests


def _declared_functions():
    with open(fa.HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) >= {"attn_fwd", "attn_fwd_cfg", "attn_fwd_plan", "fattn_strerror",
                          "fattn_version", "fattn_release"}
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n
        assert hasattr(fa.lib, n)
    # nothing else: the internal launchers and the measurement probes stay out of the ABI
    assert exported == set(names), sorted(exported - set(names))


def test_version_and_strerror():
    assert fa.fattn_version() >= 10000
    for code in (OK, INVALID, UNSUPPORTED, fa.FATTN_ERR_HIP, fa.FATTN_ERR_NOMEM):
        assert fa.fattn_strerror(code) != fa.fattn_strerror(12345)
    assert fa.fattn_strerror(OK) == "ok"


def _call(**kw):
    a = dict(Q=P, K=P, V=P, O=P, LSE=P, B=1, Hq=8, Hkv=2, Tq=64, Tk=64, d=64, causal=1,
             scale=0.125, dtype=BF16, stream=None)
    a.update(kw)
    return fa.attn_fwd_raw(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["Hq"], a["Hkv"],
                           a["Tq"], a["Tk"], a["d"], a["causal"], a["scale"], a["dtype"],
                           a["stream"], kw.get("cfg"), kw.get("window"))


@pytest.mark.parametrize("kw", [
    dict(window=0), dict(window=-5), dict(window=8, Q=None), dict(window=8, Tq=65, Tk=64),
    dict(window=8, Hkv=3), dict(window=8, O=P + 2), dict(window=0, cfg=dict(block_kv=64)),
])
def test_window_invalid_arguments(kw):
    assert _call(**kw) == INVALID


@pytest.mark.parametrize("kw", [dict(window=16, B=0), dict(window=1, Tq=0),
                                dict(window=3, B=0, Q=None, K=None, V=None, O=None, LSE=None)])
def test_window_empty_problems_are_noops(kw):
    assert _call(**kw) == OK


def test_window_unsupported_head_dim():
    assert _call(window=16, d=96) == UNSUPPORTED


def test_python_binding_rejects_a_noncausal_window():
    with pytest.raises(ValueError):
        fa.attn_fwd(None, None, None, causal=False, window=4)


@pytest.mark.parametrize("kw", [
    dict(Q=None), dict(K=None), dict(V=None), dict(O=None), dict(LSE=None),
    dict(Q=P + 2), dict(K=P + 8), dict(O=P + 4), dict(LSE=P + 1),
    dict(B=-1), dict(Hq=-2), dict(Tq=-1), dict(Tk=-1), dict(d=-64),
    dict(Hkv=0), dict(Hkv=3), dict(Tk=0), dict(d=0),
    dict(causal=2), dict(causal=-1), dict(Tq=65, Tk=64, causal=1),
    dict(scale=float("nan")), dict(scale=float("inf")), dict(dtype=7),
    dict(Tq=1 << 30, Tk=1 << 30, causal=0, d=64),
])
def test_invalid_arguments(kw):
    assert _call(**kw) == INVALID


@pytest.mark.parametrize("d", [16, 48, 96, 256])
def test_unsupported_head_dims(d):
    assert _call(d=d) == UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=0), dict(Tq=0), dict(Hq=0, Hkv=0),
                                dict(B=0, Q=None, K=None, V=None, O=None, LSE=None)])
def test_empty_problems_are_noops(kw):
    assert _call(**kw) == OK


@pytest.mark.parametrize("cfg", [dict(block_kv=48), dict(waves=2), dict(waves=16),
                                 dict(schedule=9), dict(schedule=3), dict(schedule=4, waves=4),
                                 dict(kernel=99),
                                 dict(kernel=3),
                                 dict(kernel=2), dict(splits=4), dict(block_q=64)])
def test_unsupported_configs(cfg):
    assert fa.lib.attn_fwd_plan(1, 8, 2, 64, 64, 64, 1, BF16, ctypes.byref(fa._make_cfg(cfg)),
                                ctypes.byref(fa.FattnCfg())) == UNSUPPORTED


def test_plan_defaults():
    p = fa.attn_fwd_plan(1, 32, 32, 8192, 8192, 128, True, BF16)
    assert p["kernel"] == fa.FATTN_KERNEL_PREFILL_MFMA
    assert p["block_q"] == 32 * p["waves"] and p["block_kv"] in (32, 64)
    p = fa.attn_fwd_plan(1, 4, 4, 128, 128, 32, True, F32)
    assert p["kernel"] == fa.FATTN_KERNEL_PREFILL_F32
    p = fa.attn_fwd_plan(64, 64, 8, 1, 8192, 128, False, BF16)
    assert p["kernel"] == fa.FATTN_KERNEL_DECODE_SPLITK
    assert 1 <= p["splits"] <= 8192 // 32
    # every split holds at least one key and together they cover all keys
    chunk = -(-(-(-8192 // p["splits"])) // 32) * 32
    assert (p["splits"] - 1) * chunk < 8192 <= p["splits"] * chunk


@pytest.mark.parametrize("Tk", [1, 31, 32, 33, 100, 1000, 8192, 100000])
@pytest.mark.parametrize("splits", [0, 1, 3, 7, 64, 5000])
def test_decode_split_geometry(Tk, splits):
    p = fa.attn_fwd_plan(2, 16, 2, 1, Tk, 64, False, BF16, dict(splits=splits))
    s = p["splits"]
    assert 1 <= s <= max(1, -(-Tk // 32))
    if splits:
        assert s <= splits


def test_plan_overrides_and_causal_decode():
    p = fa.attn_fwd_plan(1, 8, 8, 256, 256, 64, False, BF16, dict(block_kv=32, waves=8, schedule=1))
    assert (p["block_kv"], p["waves"], p["block_q"], p["schedule"]) == (32, 8, 256, 1)
    # a causal single query row sees every key: the decode path serves it
    p = fa.attn_fwd_plan(1, 8, 2, 1, 77, 128, True, BF16)
    assert p["kernel"] == fa.FATTN_KERNEL_DECODE_SPLITK
    # the MFMA prefill kernel also serves Tq == 1 when asked for
    p = fa.attn_fwd_plan(1, 8, 2, 1, 77, 128, True, BF16, dict(kernel=1))
    assert p["kernel"] == fa.FATTN_KERNEL_PREFILL_MFMA


def test_python_binding_raises_with_code():
    with pytest.raises(fa.FattnError) as e:
        fa.attn_fwd_plan(1, 8, 3, 64, 64, 64, True, BF16)
    assert e.value.code == INVALID
    assert "multiple of Hkv" in e.value.detail


def test_last_error_text_follows_each_call():
    assert _call(d=96) == UNSUPPORTED and "96" in fa.fattn_last_error()
    assert _call(Q=P + 2) == INVALID and "aligned" in fa.fattn_last_error()
    assert _call(B=0) == OK and fa.fattn_last_error() == ""


def test_python_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.attn_fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.attn_fwd(q.half(), q.half(), q.half())


def test_probe_library_rejects_invalid_arguments():
    # the benchmark's measurement probes live in their own library; invalid arguments are refused
    # before any HIP call
    import os

    plib = ctypes.CDLL(os.path.join(os.path.dirname(fa.__file__), "libfattn_probe.so"))
    plib.probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    plib.probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_void_p]
    for args in [(None, 1, 1, 0), (P, 0, 1, 0), (P, 1, 0, 0), (P, 1, 1, 2), (P, 1, 1, -1)]:
        assert plib.probe_mfma_bf16(*args, None) == -1
    for args in [(None, 16, P, 1), (P, 8, P, 1), (P, 24, P, 1), (P + 4, 16, P, 1),
                 (P, 16, None, 1), (P, 16, P, 0)]:
        assert plib.probe_hbm_read(*args, None) == -1
