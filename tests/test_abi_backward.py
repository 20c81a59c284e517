"""C-ABI checks of attn_bwd that need no GPU: argument errors, unsupported forms, no-ops.

Every call here has an invalid argument or no work, so the library returns before any HIP call.
"""

import pytest

import io_aware_tiled_amd as fa

OK, INVALID, UNSUPPORTED = fa.FATTN_OK, fa.FATTN_ERR_INVALID, fa.FATTN_ERR_UNSUPPORTED
BF16, F32 = fa.FATTN_BF16, fa.FATTN_F32
P = 0x10000  # a 16-byte aligned stand-in pointer; never dereferenced in these tests
PTRS = ("Q", "K", "V", "O", "dO", "LSE", "dQ", "dK", "dV")


def _call(**kw):
    a = dict(B=1, Hq=8, Hkv=2, Tq=64, Tk=64, d=64, causal=1, window=0, scale=0.125, dtype=BF16,
             stream=None)
    a.update({n: P for n in PTRS})
    a.update(kw)
    return fa.attn_bwd_raw(*(a[n] for n in PTRS), a["B"], a["Hq"], a["Hkv"], a["Tq"], a["Tk"],
                           a["d"], a["causal"], a["window"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [{n: None} for n in PTRS] + [{n: P + 4} for n in PTRS] + [
    dict(B=-1), dict(Hq=-1), dict(Tq=-3), dict(Tk=-1), dict(d=-64), dict(Hkv=0), dict(Hkv=3),
    dict(Tk=0), dict(d=0), dict(causal=2), dict(Tq=65, Tk=64),
    dict(scale=float("nan")), dict(scale=float("-inf")), dict(dtype=5),
    dict(window=-1), dict(window=8, causal=0),
])
def test_invalid_arguments(kw):
    assert _call(**kw) == INVALID, fa.fattn_last_error()


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(dtype=F32)])
def test_unsupported(kw):
    assert _call(**kw) == UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=0), dict(Tq=0), dict(Hq=0, Hkv=0),
                                dict(B=0, **{n: None for n in PTRS})])
def test_empty_problems_are_noops(kw):
    assert _call(**kw) == OK


def test_error_text():
    assert _call(dtype=F32) == UNSUPPORTED and "bf16" in fa.fattn_last_error()
    assert _call(window=4, causal=0) == INVALID and "causal" in fa.fattn_last_error()


def test_python_binding_checks():
    import torch

    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        fa.attn_bwd(q, q, q, q, lse, q, causal=False, window=4)
    with pytest.raises(ValueError):
        fa.attn_bwd(q, q, q, q, lse, q)  # CPU tensors
    with pytest.raises(TypeError):
        fa.attn_bwd(q.float(), q, q, q, lse, q)
