"""Measurement kernels: the copy and fill kernels move the right bytes."""

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_copy_fill_read(lib):
    n = (1 << 24) + 16 * 37
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    lib.util_copy(src, dst, n)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    lib.util_fill(dst, n, 0x01020304)
    torch.cuda.synchronize()
    assert torch.equal(dst.view(torch.int32), torch.full((n // 4,), 0x01020304, dtype=torch.int32,
                                                          device="cuda"))
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    lib.util_read(src, n, sink)
    torch.cuda.synchronize()
    assert lib.num_cus() > 0
