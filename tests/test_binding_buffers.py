"""The binding's checks of caller-supplied output buffers (CPU only, nothing is launched).

A buffer of the wrong shape, dtype or layout, or on another device, must be refused before the C
call: the kernels write every element of the expected shape at contiguous offsets.
"""

import pytest
import torch

import io_aware_tiled_amd as fa

CPU = torch.device("cpu")


def test_a_matching_buffer_passes():
    fa.check_out("out", torch.empty(2, 4, 8, 16), (2, 4, 8, 16), torch.float32, CPU)


@pytest.mark.parametrize("buf,err", [
    (torch.empty(2, 4, 8, 15), ValueError),                          # short last dim
    (torch.empty(2, 4, 7, 16), ValueError),                          # short rows
    (torch.empty(2 * 4 * 8 * 16), ValueError),                       # flat, right size
    (torch.empty(2, 4, 8, 16, dtype=torch.bfloat16), TypeError),     # wrong dtype
    (torch.empty(2, 4, 16, 8).transpose(2, 3), ValueError),         # strided view
    (torch.empty(2, 4, 8, 32)[..., :16], ValueError),               # sliced view
])
def test_a_mismatched_buffer_is_refused(buf, err):
    with pytest.raises(err):
        fa.check_out("out", buf, (2, 4, 8, 16), torch.float32, CPU)


def test_a_buffer_on_another_device_is_refused():
    with pytest.raises(ValueError):
        fa.check_out("lse", torch.empty(3, 5), (3, 5), torch.float32, torch.device("cuda:0"))


def test_the_lse_must_be_float32():
    with pytest.raises(TypeError):
        fa.check_out("lse", torch.empty(3, 5, dtype=torch.float64), (3, 5), torch.float32, CPU)
