"""The device e4m3 cast (the quantiser's quant4, through llt_e4m3_cast) against the oracle's C
emulator (oracle/e4m3_cast.c) on every one of the 2^32 fp32 bit patterns at scale 1, and on every
61st pattern at other power-of-two scales: codes bit-exact, NaN products 0x7F, infinities and
overflowing products clamped to +-448."""
import numpy as np
import pytest
import torch

from oracle import e4m3_c
from tests.gpu_util import need_gpu
from transformer_train_step_amd import _lib as L

pytestmark = pytest.mark.gpu

CH = 1 << 28


def test_e4m3_cast_every_fp32_pattern():
    need_gpu()
    x = torch.empty(CH, dtype=torch.int32, device="cuda")
    q = torch.empty(CH, dtype=torch.uint8, device="cuda")
    ramp = torch.arange(CH, dtype=torch.int32, device="cuda")
    for first in range(0, 1 << 32, CH):
        print(f"e4m3 cast: patterns {first:#010x} .. {first + CH - 1:#010x}", flush=True)
        x.copy_(ramp).add_(first if first < (1 << 31) else first - (1 << 32))   # two's complement bits
        L.llt_e4m3_cast(x.view(torch.float32), CH, 1.0, q)
        got = q.cpu().numpy()
        ref = e4m3_c.cast_patterns(first, CH, 1.0, threads=16)
        if not np.array_equal(got, ref):
            i = int(np.flatnonzero(got != ref)[0])
            raise AssertionError(f"pattern {first + i:#010x}: device {int(got[i]):#04x}, oracle {int(ref[i]):#04x} "
                                 f"({int((got != ref).sum())} codes differ in this chunk)")


@pytest.mark.parametrize("scale", [2.0 ** -7, 2.0 ** 5, 2.0 ** 40])
def test_e4m3_cast_scaled_patterns(scale):
    need_gpu()
    print(f"e4m3 cast at scale {scale}", flush=True)
    bits = np.arange(0, (1 << 32) // 61, dtype=np.uint32) * np.uint32(61)
    n = bits.size - bits.size % 4
    xs = bits[:n].view(np.float32)
    xd = torch.from_numpy(xs.view(np.int32)).cuda()
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    L.llt_e4m3_cast(xd.view(torch.float32), n, scale, q)
    assert np.array_equal(q.cpu().numpy(), e4m3_c.cast(xs, scale))


def test_e4m3_cast_validates():
    need_gpu()
    x = torch.zeros(8, dtype=torch.float32, device="cuda")
    q = torch.empty(8, dtype=torch.uint8, device="cuda")
    assert L.llt_e4m3_cast(x, 6, 1.0, q, raise_on_error=False) != 0     # n not a multiple of 4
    assert L.llt_e4m3_cast(x, 0, 1.0, q) == 0
