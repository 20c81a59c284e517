"""C-ABI checks of attn_fwd_paged that need no GPU: argument errors, unsupported forms, no-ops.

Every call here has an invalid argument or no work, so the library returns before any HIP call.
"""

import pytest

import io_aware_tiled_amd as fa

OK, INVALID, UNSUPPORTED = fa.FATTN_OK, fa.FATTN_ERR_INVALID, fa.FATTN_ERR_UNSUPPORTED
BF16, F32 = fa.FATTN_BF16, fa.FATTN_F32
P = 0x10000  # a 16-byte aligned stand-in pointer; never dereferenced in these tests
PTRS = ("Q", "Kc", "Vc", "table", "lens", "O", "LSE")


def _call(**kw):
    a = dict(B=2, Hq=8, Hkv=2, d=128, num_blocks=64, bs=16, max_blocks=32, scale=0.1,
             dtype=BF16, stream=None)
    a.update({n: P for n in PTRS})
    a.update(kw)
    return fa.attn_fwd_paged_raw(*(a[n] for n in PTRS), a["B"], a["Hq"], a["Hkv"], a["d"],
                                 a["num_blocks"], a["bs"], a["max_blocks"], a["scale"],
                                 a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [{n: None} for n in PTRS] + [
    dict(Q=P + 8), dict(Kc=P + 2), dict(Vc=P + 4), dict(O=P + 8), dict(LSE=P + 4),
    dict(table=P + 2), dict(lens=P + 1),
    dict(bs=8), dict(bs=24), dict(bs=8192), dict(bs=0), dict(num_blocks=0),
    dict(max_blocks=0), dict(max_blocks=1 << 28, bs=4096),
    dict(B=-1), dict(Hq=-8), dict(Hkv=0), dict(Hkv=3), dict(d=0),
    dict(scale=float("nan")), dict(dtype=9),
])
def test_invalid_arguments(kw):
    assert _call(**kw) == INVALID, fa.fattn_last_error()


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(dtype=F32)])
def test_unsupported(kw):
    assert _call(**kw) == UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=0), dict(Hq=0, Hkv=0),
                                dict(B=0, **{n: None for n in PTRS})])
def test_empty_problems_are_noops(kw):
    assert _call(**kw) == OK


def test_error_text():
    assert _call(bs=48) == INVALID and "power of two" in fa.fattn_last_error()


def test_python_binding_checks():
    import torch

    q = torch.zeros(2, 8, 64, dtype=torch.bfloat16)
    kc = torch.zeros(4, 2, 16, 64, dtype=torch.bfloat16)
    t = torch.zeros(2, 2, dtype=torch.int32)
    n = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        fa.attn_fwd_paged(q, kc, kc, t, n)  # CPU tensors
    with pytest.raises(TypeError):
        fa.attn_fwd_paged(q, kc, kc, t.long(), n)
