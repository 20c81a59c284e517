"""The benchmark's own work formulas agree with the oracle's accounting (CPU only)."""

import pytest

import bench
from oracle import accounting as acc


@pytest.mark.parametrize("shape", [(1, 32, 8192, 8192, 128, True), (4, 16, 1024, 1024, 64, True),
                                   (1, 32, 4096, 4096, 128, False)])
def test_prefill_flops(shape):
    B, H, Tq, Tk, d, causal = shape
    assert bench.prefill_flops(B, H, Tq, Tk, d, causal) == acc.attention_flops(B, H, Tq, Tk, d,
                                                                               causal)


def test_decode_bytes():
    assert bench.decode_bytes(64, 64, 8, 8192, 128) == acc.decode_bytes(64, 64, 8, 8192, 128)


@pytest.mark.parametrize("T,W", [(10, 3), (5, 10), (257, 64), (1000, 1), (64, 64)])
def test_window_pairs(T, W):
    assert bench.window_pairs(T, W) == acc.visible_pairs(T, T, True, W)


def test_window_decode_bytes_read_only_the_window():
    assert bench.window_decode_bytes(64, 64, 8, 4096, 128) == acc.decode_bytes(64, 64, 8, 4096,
                                                                               128)


@pytest.mark.parametrize("shape", [(1, 32, 8192, 8192, 128, True), (2, 8, 300, 300, 64, False)])
def test_backward_flops(shape):
    import oracle

    assert bench.backward_flops(*shape) == oracle.backward_flops(*shape)
    B, H, Tq, Tk, d, causal = shape
    # five products against the forward's two: 2.5 times the forward count
    assert bench.backward_flops(*shape) == 2.5 * bench.prefill_flops(B, H, Tq, Tk, d, causal)


def test_varlen_document_lengths_cover_the_batch():
    lens = bench.varlen_doc_lengths(bench.VARLEN_TOKENS, 128, 8192, bench.VARLEN_SEED)
    assert sum(lens) == bench.VARLEN_TOKENS and all(1 <= n <= 8192 for n in lens)
    # the work counted is each document's causal count, as the oracle's accounting has it
    total = sum(bench.prefill_flops(1, 32, n, n, 128, True) for n in lens)
    assert total == sum(acc.attention_flops(1, 32, n, n, 128, True) for n in lens)
