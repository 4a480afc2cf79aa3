"""GPU checks of moe_finalize_rmsnorm_checked and moe_finalize_rmsnorm_fp8_checked,
the fused op (bf16 or FP8 output) told the row count R of expert_out: in-range
indices give the plain op's outputs bit for bit and leave the flag clear; an
index at or past R is treated as masked and raises the flag."""
import numpy as np
import pytest
import torch

import synth
import top_finalize_residual_amd as mfr
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _args(dd):
    return [dd[k] for k in ("expert_out", "perm_idx", "topk_w", "shared_out", "residual", "gamma")]


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
@pytest.mark.parametrize("cfg,T", [("decode", 28), ("decode_masked", 64), ("batch512", 512)])
def test_in_range_equals_plain_call(cfg, T, path):
    d = synth.config_inputs(cfg, T)
    dd = gu.to_device(d)
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=path)
    with gu.forced(path, 0, 0):
        r, n, bad = mfr.moe_finalize_rmsnorm_checked(*_args(dd), d["eps"], d["scale"])
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_u16(r), r0) and np.array_equal(gu.host_u16(n), n0)
    assert int(bad.item()) == 0


@pytest.mark.parametrize("K", [8, 12], ids=["K8", "K12"])
@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_rows_past_r_are_masked_and_reported(path, K):
    """expert_out holds more rows than the R it is declared with, so the
    slots whose index lies in [R, T*K) point at real memory. The checked
    call must treat them as masked, which equals the plain call with those
    indices set to -1, and raise the flag."""
    T, H = 64, 2048
    d = synth.generate(T, H, K, scale=2.5, mask_frac=0.05, seed=810 + K, extra_rows=16)
    R = T * K - 40
    dd = gu.to_device(d)
    declared = dd["expert_out"][:R]
    past = d["perm_idx"] >= R
    assert past.any() and (d["perm_idx"] < 0).any()
    masked = d["perm_idx"].copy()
    masked[past] = -1
    dm = dict(dd, perm_idx=torch.from_numpy(masked).cuda())
    r0, n0 = gu.run(dm, d["eps"], d["scale"], path=path)
    with gu.forced(path, 0, 0):
        r, n, bad = mfr.moe_finalize_rmsnorm_checked(declared, *_args(dd)[1:], d["eps"], d["scale"])
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_u16(r), r0) and np.array_equal(gu.host_u16(n), n0)
    assert int(bad.item()) == 1
    # the same without a flag: the C call with bad_index = NULL
    ro, no = torch.empty_like(dd["residual"]), torch.empty_like(dd["residual"])
    a = [t.data_ptr() for t in _args(dd)]
    with gu.forced(path, 0, 0):
        rc = mfr.binding.lib().moe_finalize_rmsnorm_checked(
            a[0], R, *a[1:], d["eps"], d["scale"], ro.data_ptr(), no.data_ptr(), None, T, H, K,
            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert np.array_equal(gu.host_u16(ro), r0) and np.array_equal(gu.host_u16(no), n0)


def test_far_index_is_masked_not_read():
    """Indices far past the rows (up to 2^31 - 1) touch no memory: the slot
    is masked, the outputs equal the plain call with the slot set to -1, and
    the flag is raised. Tokens with no such index are unaffected."""
    T, H, K = 16, 2048, 8
    d = synth.generate(T, H, K, scale=2.5, seed=820)
    dd = gu.to_device(d)
    bad = d["perm_idx"].copy()
    bad[3, 2] = 2 ** 31 - 1
    bad[9, 7] = T * K + 123456
    masked = bad.copy()
    masked[3, 2] = -1
    masked[9, 7] = -1
    r0, n0 = gu.run(dict(dd, perm_idx=torch.from_numpy(masked).cuda()), d["eps"], d["scale"])
    r, n, flag = mfr.moe_finalize_rmsnorm_checked(dd["expert_out"], torch.from_numpy(bad).cuda(),
                                                  *_args(dd)[2:], d["eps"], d["scale"])
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_u16(r), r0) and np.array_equal(gu.host_u16(n), n0)
    assert int(flag.item()) == 1


# --- the FP8-output form ---------------------------------------------------

def _fp8_plain(dd, d, perm_idx=None):
    r, q, s, n = mfr.moe_finalize_rmsnorm_fp8(dd["expert_out"],
                                              dd["perm_idx"] if perm_idx is None else perm_idx,
                                              *_args(dd)[2:], d["eps"], d["scale"],
                                              bf16_normed=True)
    torch.cuda.synchronize()
    return r, q, s, n


def _same(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
@pytest.mark.parametrize("cfg,T", [("decode", 28), ("decode_masked", 64), ("batch512", 512)])
def test_fp8_in_range_equals_plain_fp8_call(cfg, T, path):
    d = synth.config_inputs(cfg, T)
    dd = gu.to_device(d)
    with gu.forced(path, 0, 0):
        want = _fp8_plain(dd, d)
        r, q, s, n, bad = mfr.moe_finalize_rmsnorm_fp8_checked(*_args(dd), d["eps"], d["scale"],
                                                               bf16_normed=True)
    torch.cuda.synchronize()
    assert _same((r, q, s, n), want)
    assert int(bad.item()) == 0


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_fp8_rows_past_r_are_masked_and_reported(path):
    """As for the bf16 form: the rows in [R, T*K) are real memory, and the
    checked FP8 call equals the plain FP8 call with those slots set to -1."""
    T, H, K = 64, 2048, 12
    d = synth.generate(T, H, K, scale=2.5, mask_frac=0.05, seed=830, extra_rows=16)
    R = T * K - 40
    dd = gu.to_device(d)
    past = d["perm_idx"] >= R
    assert past.any()
    masked = d["perm_idx"].copy()
    masked[past] = -1
    with gu.forced(path, 0, 0):
        want = _fp8_plain(dd, d, torch.from_numpy(masked).cuda())
        r, q, s, n, bad = mfr.moe_finalize_rmsnorm_fp8_checked(dd["expert_out"][:R],
                                                               *_args(dd)[1:], d["eps"],
                                                               d["scale"], bf16_normed=True)
    torch.cuda.synchronize()
    assert _same((r, q, s, n), want)
    assert int(bad.item()) == 1


def test_fp8_far_index_is_masked_not_read():
    T, H, K = 16, 2048, 8
    d = synth.generate(T, H, K, scale=2.5, seed=840)
    dd = gu.to_device(d)
    bad_idx = d["perm_idx"].copy()
    bad_idx[5, 1] = 2 ** 31 - 1
    masked = bad_idx.copy()
    masked[5, 1] = -1
    want = _fp8_plain(dd, d, torch.from_numpy(masked).cuda())
    r, q, s, n, flag = mfr.moe_finalize_rmsnorm_fp8_checked(
        dd["expert_out"], torch.from_numpy(bad_idx).cuda(), *_args(dd)[2:], d["eps"], d["scale"],
        bf16_normed=True)
    torch.cuda.synchronize()
    assert _same((r, q, s, n), want)
    assert int(flag.item()) == 1


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_zero_rows(fp8):
    """R = 0 (an empty expert_out): every slot is past the rows, so each is
    masked and flagged; the outputs equal the plain call with every slot
    masked. With every index already negative, the flag stays clear."""
    T, H, K = 12, 2048, 8
    d = synth.generate(T, H, K, scale=2.5, seed=850)
    dd = gu.to_device(d)
    empty = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    all_masked = torch.full((T, K), -1, dtype=torch.int32, device="cuda")
    for idx, flag in ((dd["perm_idx"], 1), (all_masked, 0)):
        if fp8:
            want = _fp8_plain(dd, d, all_masked)
            r, q, s, n, bad = mfr.moe_finalize_rmsnorm_fp8_checked(
                empty, idx, *_args(dd)[2:], d["eps"], d["scale"], bf16_normed=True)
            got = (r, q, s, n)
        else:
            want = gu.run(dict(dd, perm_idx=all_masked), d["eps"], d["scale"])
            r, n, bad = mfr.moe_finalize_rmsnorm_checked(empty, idx, *_args(dd)[2:], d["eps"],
                                                         d["scale"])
            got = (r, n)
        torch.cuda.synchronize()
        if fp8:
            assert _same(got, want)
        else:
            assert np.array_equal(gu.host_u16(r), want[0]) and np.array_equal(gu.host_u16(n), want[1])
        assert int(bad.item()) == flag
