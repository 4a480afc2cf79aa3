"""The bandwidth probes behind the ceilings the benchmark reports compute what
they claim, on small buffers: the copy probe copies, and the mixed-stream
probe's every output vector is the XOR of its share of the unit's loads, in
both forms (one unit per workgroup pass, and the pipelined walk), with and
without the residency cap, and with FP8 codes the second region holds the
folded halves of those vectors. A probe that skipped loads would stream faster
than it should and inflate the ceilings."""
import ctypes

import numpy as np
import pytest
import torch

import bench

pytestmark = pytest.mark.gpu


def _mix_expected(src_u32, units, a, b):
    """Expected output (uint32 words) of the mixed-stream probe: unit u,
    output vector j, thread x is the XOR of loads j, j + b, j + 2b, ... of
    that thread in that unit."""
    v = src_u32[: units * a * 256 * 4].reshape(units, a, 256, 4)
    out = np.zeros((units, b, 256, 4), dtype=np.uint32)
    for j in range(b):
        out[:, j] = np.bitwise_xor.reduce(v[:, j::b], axis=1)
    return out.reshape(-1)


@pytest.mark.parametrize("a,b", [(30, 6), (20, 3), (10, 2), (40, 8)])
@pytest.mark.parametrize("flags,grid,per_cu", [(0, 0, 0), (1, 0, 2), (1, 5, 0), (2, 3, 0),
                                               (3, 7, 0)])
def test_mix_probe_output(a, b, flags, grid, per_cu):
    lib = bench._probe_lib()
    units = 11  # more than the grids above, so the walks take several units each
    rng = np.random.default_rng(1234 + a + 10 * flags)
    src = rng.integers(0, 2**32, size=units * a * 256 * 4 + 4 * 256, dtype=np.uint32)
    d_src = torch.from_numpy(src.view(np.int32)).cuda()
    d_dst = torch.zeros(units * b * 256 * 4 + 4 * 256, dtype=torch.int32, device="cuda")
    rb, wb = ctypes.c_int64(0), ctypes.c_int64(0)
    rc = lib.mfr_mix_probe(d_src.data_ptr(), units * a * 4096, d_dst.data_ptr(),
                           units * b * 4096, a, b, flags, grid, per_cu, ctypes.byref(rb),
                           ctypes.byref(wb), torch.cuda.current_stream().cuda_stream)
    if rc == 3:
        pytest.skip("this residency cannot be set through LDS for this kernel")
    assert rc == 0
    torch.cuda.synchronize()
    assert rb.value == units * a * 4096 and wb.value == units * b * 4096
    got = d_dst.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got[: units * b * 1024], _mix_expected(src, units, a, b))
    assert not got[units * b * 1024:].any()  # nothing written past the units


@pytest.mark.parametrize("flags,grid,per_cu", [(4, 0, 0), (5, 0, 2), (5, 5, 0), (6, 3, 0),
                                               (7, 7, 0)])
def test_mix_probe_codes_form(flags, grid, per_cu):
    """The FP8-code form, pair (30, 3): per unit, three 16-byte vectors per
    thread in the first region, then three 8-byte ones (each vector's halves
    XORed together) in the second, which starts where the units' 16-byte
    writes end."""
    lib = bench._probe_lib()
    a, b, units = 30, 3, 11
    rng = np.random.default_rng(4321 + flags)
    src = rng.integers(0, 2**32, size=units * a * 256 * 4 + 4 * 256, dtype=np.uint32)
    d_src = torch.from_numpy(src.view(np.int32)).cuda()
    w16 = units * b * 256 * 4  # words of the first region
    d_dst = torch.zeros(w16 + w16 // 2 + 4 * 256, dtype=torch.int32, device="cuda")
    rb, wb = ctypes.c_int64(0), ctypes.c_int64(0)
    rc = lib.mfr_mix_probe(d_src.data_ptr(), units * a * 4096, d_dst.data_ptr(),
                           (w16 + w16 // 2) * 4, a, b, flags, grid, per_cu, ctypes.byref(rb),
                           ctypes.byref(wb), torch.cuda.current_stream().cuda_stream)
    if rc == 3:
        pytest.skip("this residency cannot be set through LDS for this kernel")
    assert rc == 0
    torch.cuda.synchronize()
    assert rb.value == units * a * 4096 and wb.value == units * b * 4096 * 3 // 2
    got = d_dst.cpu().numpy().view(np.uint32)
    x = _mix_expected(src, units, a, b)
    np.testing.assert_array_equal(got[:w16], x)
    x4 = x.reshape(-1, 4)
    halves = np.stack([x4[:, 0] ^ x4[:, 2], x4[:, 1] ^ x4[:, 3]], axis=1).reshape(-1)
    np.testing.assert_array_equal(got[w16: w16 + w16 // 2], halves)
    assert not got[w16 + w16 // 2:].any()  # nothing written past the units


def test_copy_probe_copies():
    lib = bench._probe_lib()
    n = (1 << 20) + 4096
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    assert lib.mfr_copy_probe(src.data_ptr(), dst.data_ptr(), n, 7,
                              torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
