"""C-ABI checks of attn_fwd_varlen that need no GPU: argument errors, unsupported forms, no-ops.

Every call here has an invalid argument or no work, so the library returns before any HIP call.
"""

import pytest

import io_aware_tiled_amd as fa

OK, INVALID, UNSUPPORTED = fa.FATTN_OK, fa.FATTN_ERR_INVALID, fa.FATTN_ERR_UNSUPPORTED
BF16, F32 = fa.FATTN_BF16, fa.FATTN_F32
P = 0x10000  # a 16-byte aligned stand-in pointer; never dereferenced in these tests
PTRS = ("Q", "K", "V", "O", "LSE", "cu_q", "cu_k")


def _call(**kw):
    a = dict(n=3, total_q=300, total_k=300, max_q=200, max_k=200, Hq=8, Hkv=2, d=64, causal=1,
             window=0, scale=0.125, dtype=BF16, stream=None)
    a.update({n: P for n in PTRS})
    a.update(kw)
    return fa.attn_fwd_varlen_raw(*(a[n] for n in PTRS), a["n"], a["total_q"], a["total_k"],
                                  a["max_q"], a["max_k"], a["Hq"], a["Hkv"], a["d"], a["causal"],
                                  a["window"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [{n: None} for n in PTRS] + [
    dict(Q=P + 2), dict(K=P + 8), dict(V=P + 4), dict(O=P + 2), dict(LSE=P + 4),
    dict(cu_q=P + 2), dict(cu_k=P + 1),
    dict(n=-1), dict(total_q=-1), dict(total_k=-5), dict(max_q=-1), dict(max_k=-1),
    dict(Hq=-8), dict(Hkv=0), dict(Hkv=3), dict(d=0), dict(causal=2),
    dict(window=-1), dict(window=16, causal=0), dict(scale=float("inf")), dict(dtype=3),
])
def test_invalid_arguments(kw):
    assert _call(**kw) == INVALID, fa.fattn_last_error()


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=256), dict(dtype=F32)])
def test_unsupported(kw):
    assert _call(**kw) == UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(n=0), dict(total_q=0), dict(Hq=0, Hkv=0),
                                dict(n=0, **{n: None for n in PTRS})])
def test_empty_problems_are_noops(kw):
    assert _call(**kw) == OK


def test_causal_with_more_queries_than_keys_is_allowed_on_the_host():
    # per-document lengths are device data; such rows get O = 0, LSE = -inf in the kernel
    assert _call(max_q=300, max_k=100, d=96) == UNSUPPORTED  # reaches the head-dim check


def test_python_binding_checks():
    import torch

    q = torch.zeros(10, 4, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError):
        fa.attn_fwd_varlen(q, q, q, cu, cu, 10, 10)  # CPU tensors
    with pytest.raises(TypeError):
        fa.attn_fwd_varlen(q, q, q, cu.long(), cu, 10, 10)
    with pytest.raises(ValueError):
        fa.attn_fwd_varlen(q, q, q, cu, cu, 10, 10, causal=False, window=3)


BPTRS = ("Q", "K", "V", "O", "dO", "LSE", "dQ", "dK", "dV", "cu_q", "cu_k")


def _bcall(**kw):
    a = dict(n=3, total_q=300, total_k=300, max_q=200, max_k=200, Hq=8, Hkv=2, d=64, causal=1,
             window=0, scale=0.125, dtype=BF16, stream=None)
    a.update({n: P for n in BPTRS})
    a.update(kw)
    return fa.attn_bwd_varlen_raw(*(a[n] for n in BPTRS), a["n"], a["total_q"], a["total_k"],
                                  a["max_q"], a["max_k"], a["Hq"], a["Hkv"], a["d"], a["causal"],
                                  a["window"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [{n: None} for n in BPTRS] + [
    dict(dQ=P + 2), dict(dK=P + 8), dict(LSE=P + 4), dict(cu_k=P + 2),
    dict(n=-1), dict(total_q=-1), dict(Hkv=3), dict(causal=2), dict(window=-1),
    dict(window=4, causal=0), dict(scale=float("nan")), dict(total_q=1 << 26, Hq=8),
])
def test_backward_invalid_arguments(kw):
    assert _bcall(**kw) == INVALID, fa.fattn_last_error()


@pytest.mark.parametrize("kw", [dict(d=96), dict(dtype=F32)])
def test_backward_unsupported(kw):
    assert _bcall(**kw) == UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(n=0), dict(total_q=0), dict(n=0, **{n: None for n in BPTRS})])
def test_backward_empty_problems_are_noops(kw):
    assert _bcall(**kw) == OK
