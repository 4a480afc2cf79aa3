"""The C ABI on the host: symbols, status codes, path query and argument
validation. Every call here returns before anything is enqueued on a GPU
(validation runs on the host first), so these run without a GPU."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

mfr = pytest.importorskip("top_finalize_residual_amd", reason="HIP library not built")
from top_finalize_residual_amd import binding  # noqa: E402
from top_finalize_residual_amd import tuning  # noqa: E402

T, H, K = 4, 2048, 8
A = 1 << 20  # fake, 16-byte aligned, never dereferenced addresses


def declared_functions():
    names = []
    for fn in sorted(os.listdir(INCLUDE)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*([A-Za-z_]\w*)\s*\(", text, re.M):
            names.append(m.group(1))
    return names


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("moe_finalize_rmsnorm", "moe_finalize_rmsnorm_path",
                 "moe_finalize_rmsnorm_strerror",
                 "residual_add_rmsnorm", "moe_finalize_rmsnorm_fp8",
                 "moe_finalize_rmsnorm_checked", "residual_add_rmsnorm_fp8",
                 "moe_finalize_rmsnorm_fp8_checked"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared but not exported"


def test_strerror_covers_every_status():
    seen = set()
    for code in range(0, 8):
        msg = mfr.strerror(code)
        assert msg and msg != "unknown status"
        seen.add(msg)
    assert len(seen) == 8
    assert mfr.strerror(99) == "unknown status"


def test_path_query():
    assert mfr.moe_finalize_rmsnorm_path(1, 6144, 8) == mfr.PATH_TOKEN
    assert mfr.moe_finalize_rmsnorm_path(28, 6144, 8) == mfr.PATH_TOKEN
    assert mfr.moe_finalize_rmsnorm_path(8192, 6144, 8) == mfr.PATH_STREAM
    assert mfr.moe_finalize_rmsnorm_path(256, 6144, 8) == mfr.PATH_TOKEN
    assert mfr.moe_finalize_rmsnorm_path(511, 6144, 8) == mfr.PATH_TOKEN
    assert mfr.moe_finalize_rmsnorm_path(512, 6144, 8) == mfr.PATH_STREAM
    assert mfr.moe_finalize_rmsnorm_path(512, 6144, 8) == mfr.PATH_STREAM
    assert mfr.moe_finalize_rmsnorm_path(0, 6144, 8) == mfr.PATH_TOKEN
    for bad in ((-1, 6144, 8), (4, 6143, 8), (4, 0, 8), (4, 16392, 8), (4, 6144, 0),
                (4, 6144, 17), (2**31, 6144, 8)):
        assert mfr.moe_finalize_rmsnorm_path(*bad) == mfr.PATH_UNSUPPORTED, bad
    assert mfr.moe_finalize_rmsnorm_path(4, 16384, 16) != mfr.PATH_UNSUPPORTED
    assert mfr.moe_finalize_rmsnorm_path(4, 8, 1) != mfr.PATH_UNSUPPORTED


def test_launch_override_validates_and_is_per_thread():
    """The tuning interface's launch override: validated, and it belongs to
    the calling thread, so another thread's calls keep the automatic shape."""
    import threading
    try:
        tuning.force_launch(mfr.PATH_STREAM, 0, 0)
        assert mfr.moe_finalize_rmsnorm_path(1, 6144, 8) == mfr.PATH_STREAM
        tuning.force_launch(mfr.PATH_TOKEN, 2, 0)
        assert mfr.moe_finalize_rmsnorm_path(8192, 6144, 8) == mfr.PATH_TOKEN
        for bad in ((4, 0, 0), (-1, 0, 0), (0, 5, 0), (0, -1, 0), (0, 0, 5), (0, 0, -1)):
            with pytest.raises(mfr.MFRError) as e:
                tuning.force_launch(*bad)
            assert e.value.status == binding.MFR_ERR_ARG
        for bad in (-1, 2):
            with pytest.raises(mfr.MFRError) as e:
                tuning.force_token_order(bad)
            assert e.value.status == binding.MFR_ERR_ARG
        with pytest.raises(mfr.MFRError) as e:
            tuning.force_residency(-1)
        assert e.value.status == binding.MFR_ERR_ARG
        # a rejected override leaves the previous one in place
        assert mfr.moe_finalize_rmsnorm_path(8192, 6144, 8) == mfr.PATH_TOKEN
        seen = []
        th = threading.Thread(target=lambda: seen.append(mfr.moe_finalize_rmsnorm_path(8192, 6144, 8)))
        th.start()
        th.join()
        assert seen == [mfr.PATH_STREAM]  # the other thread is not overridden
    finally:
        tuning.force_launch(0, 0, 0)
    assert mfr.moe_finalize_rmsnorm_path(8192, 6144, 8) == mfr.PATH_STREAM


def test_forced_restores_every_knob():
    """tuning.forced nests: on exit the enclosing override is back, token
    order and residency included, and a forced() of nothing keeps it."""
    with tuning.forced(mfr.PATH_TOKEN, 2, tuning.STORE_NONTEMPORAL, residency=2,
                       order=tuning.ORDER_XCD_RANGES):
        outer = tuning._current()
        assert outer == ((mfr.PATH_TOKEN, 2, tuning.STORE_NONTEMPORAL), 2, tuning.ORDER_XCD_RANGES)
        with tuning.forced(mfr.PATH_STREAM, 0, 0, residency=1):
            assert tuning._current() == ((mfr.PATH_STREAM, 0, 0), 1, 0)
            assert mfr.moe_finalize_rmsnorm_path(1, 6144, 8) == mfr.PATH_STREAM
        assert tuning._current() == outer
        with tuning.forced():
            assert tuning._current() == outer
        assert mfr.moe_finalize_rmsnorm_path(8192, 6144, 8) == mfr.PATH_TOKEN
    assert tuning._current() == ((0, 0, 0), 0, 0)


def test_public_header_has_no_launch_override():
    """The public header declares only the op's entry points: the launch
    override lives in the library's internal tuning header."""
    names = declared_functions()
    assert not any("force" in n for n in names), names
    text = open(os.path.join(INCLUDE, "moe_finalize_rmsnorm.h")).read()
    assert "mfr_tuning" not in text and "MFR_STORE_" not in text


def _ptrs(**over):
    """A full set of distinct, aligned fake pointers (no overlaps)."""
    act = T * H * 2
    p = dict(expert_out=A, perm_idx=A + 64 * act, topk_w=A + 65 * act, shared_out=A + 66 * act,
             residual=A + 67 * act, gamma=A + 68 * act, residual_out=A + 69 * act,
             normed_out=A + 70 * act)
    p.update(over)
    return p


def call(T_=T, H_=H, K_=K, eps=1e-6, scale=2.5, **over):
    p = _ptrs(**over)
    return mfr.moe_finalize_rmsnorm_raw(p["expert_out"], p["perm_idx"], p["topk_w"],
                                        p["shared_out"], p["residual"], p["gamma"], eps, scale,
                                        p["residual_out"], p["normed_out"], T_, H_, K_, None)


@pytest.mark.parametrize("name", ["expert_out", "perm_idx", "topk_w", "shared_out", "residual",
                                  "gamma", "residual_out", "normed_out"])
def test_null_pointer(name):
    assert call(**{name: None}) == binding.MFR_ERR_NULL


@pytest.mark.parametrize("shape", [(-1, H, K), (T, 0, K), (T, 7, K), (T, 2044, K), (T, 16392, K),
                                   (T, H, 0), (T, H, 17), (T, H, -3), (2**31, H, K)])
def test_bad_shape(shape):
    assert call(*shape) == binding.MFR_ERR_SHAPE


@pytest.mark.parametrize("name,delta", [("expert_out", 8), ("shared_out", 2), ("residual", 4),
                                        ("gamma", 8), ("residual_out", 2), ("normed_out", 8),
                                        ("perm_idx", 2), ("topk_w", 1)])
def test_misaligned(name, delta):
    base = _ptrs()[name]
    assert call(**{name: base + delta}) == binding.MFR_ERR_ALIGN


@pytest.mark.parametrize("eps,scale", [(-1e-6, 1.0), (math.nan, 1.0), (math.inf, 1.0),
                                       (1e-6, math.nan), (1e-6, math.inf), (1e-6, -math.inf)])
def test_bad_scalars(eps, scale):
    assert call(eps=eps, scale=scale) == binding.MFR_ERR_SCALAR


def test_zero_tokens_is_a_no_op():
    # T == 0: accepted without launching, pointers are not examined
    assert mfr.moe_finalize_rmsnorm_raw(None, None, None, None, None, None, 1e-6, 1.0,
                                        None, None, 0, H, K, None) == binding.MFR_OK


def test_shape_checked_before_pointers():
    assert mfr.moe_finalize_rmsnorm_raw(None, None, None, None, None, None, 1e-6, 1.0,
                                        None, None, 0, 7, K, None) == binding.MFR_ERR_SHAPE


def test_aliasing_rules():
    p = _ptrs()
    act = T * H * 2
    # overlapping outputs
    assert call(normed_out=p["residual_out"]) == binding.MFR_ERR_ALIAS
    assert call(normed_out=p["residual_out"] + act - 16) == binding.MFR_ERR_ALIAS
    # residual_out partially overlapping residual
    assert call(residual_out=p["residual"] + 16) == binding.MFR_ERR_ALIAS
    # outputs on top of other inputs
    for name in ("shared_out", "gamma", "perm_idx", "topk_w", "expert_out"):
        assert call(residual_out=p[name]) == binding.MFR_ERR_ALIAS, name
        assert call(normed_out=p[name]) == binding.MFR_ERR_ALIAS, name
    assert call(normed_out=p["residual"]) == binding.MFR_ERR_ALIAS
    # in place (residual_out == residual) and touching buffers are accepted: the
    # GPU tests exercise them, since a call that passes validation launches


def dense_call(T_=T, H_=H, eps=1e-6, **over):
    act = T * H * 2
    p = dict(x=A, residual=A + 4 * act, gamma=A + 8 * act, residual_out=A + 12 * act,
             normed_out=A + 16 * act)
    p.update(over)
    return mfr.residual_add_rmsnorm_raw(p["x"], p["residual"], p["gamma"], eps, p["residual_out"],
                                        p["normed_out"], T_, H_, None)


def test_dense_validation():
    act = T * H * 2
    for name in ("x", "residual", "gamma", "residual_out", "normed_out"):
        assert dense_call(**{name: None}) == binding.MFR_ERR_NULL, name
        assert dense_call(**{name: A + 20 * act + 8}) == binding.MFR_ERR_ALIGN, name
    for shape in ((-1, H), (T, 0), (T, 12), (T, 16392), (2**31, H)):
        assert dense_call(*shape) == binding.MFR_ERR_SHAPE, shape
    for eps in (-1.0, math.nan, math.inf):
        assert dense_call(eps=eps) == binding.MFR_ERR_SCALAR
    assert dense_call(normed_out=A + 12 * act) == binding.MFR_ERR_ALIAS  # == residual_out
    assert dense_call(residual_out=A) == binding.MFR_ERR_ALIAS  # on x
    assert dense_call(normed_out=A + 4 * act + 16) == binding.MFR_ERR_ALIAS  # inside residual
    assert dense_call(residual_out=A + 4 * act + 16) == binding.MFR_ERR_ALIAS  # partial overlap
    assert dense_call(residual_out=A + 8 * act) == binding.MFR_ERR_ALIAS  # on gamma
    assert mfr.residual_add_rmsnorm_raw(None, None, None, 1e-6, None, None, 0, H, None) == binding.MFR_OK


def fp8_call(T_=T, H_=H, K_=K, **over):
    act = T * H * 2
    p = dict(_ptrs(), normed_fp8=A + 80 * act, fp8_scale=A + 90 * act)
    p.update(over)
    return mfr.moe_finalize_rmsnorm_fp8_raw(p["expert_out"], p["perm_idx"], p["topk_w"],
                                            p["shared_out"], p["residual"], p["gamma"], 1e-6, 2.5,
                                            p["residual_out"], p["normed_out"], p["normed_fp8"],
                                            p["fp8_scale"], T_, H_, K_, None)


def test_fp8_validation():
    act = T * H * 2
    base = dict(_ptrs(), normed_fp8=A + 80 * act, fp8_scale=A + 90 * act)
    for name in ("expert_out", "perm_idx", "topk_w", "shared_out", "residual", "gamma",
                 "residual_out", "normed_fp8", "fp8_scale"):
        assert fp8_call(**{name: None}) == binding.MFR_ERR_NULL, name
    assert fp8_call(normed_fp8=base["normed_fp8"] + 4) == binding.MFR_ERR_ALIGN
    assert fp8_call(fp8_scale=base["fp8_scale"] + 2) == binding.MFR_ERR_ALIGN
    assert fp8_call(normed_out=base["normed_out"] + 8) == binding.MFR_ERR_ALIGN
    assert fp8_call(T_=4, H_=12) == binding.MFR_ERR_SHAPE
    # codes on top of the residual output, the scale inside the codes, codes on an input
    assert fp8_call(normed_fp8=base["residual_out"]) == binding.MFR_ERR_ALIAS
    assert fp8_call(fp8_scale=base["normed_fp8"] + 64) == binding.MFR_ERR_ALIAS
    assert fp8_call(normed_fp8=base["shared_out"]) == binding.MFR_ERR_ALIAS
    assert fp8_call(normed_out=base["normed_fp8"]) == binding.MFR_ERR_ALIAS
    # without the optional bf16 output, its pointer is not examined
    assert fp8_call(T_=0, normed_out=None) == binding.MFR_OK


def dense_fp8_call(T_=T, H_=H, eps=1e-6, **over):
    act = T * H * 2
    p = dict(x=A, residual=A + 4 * act, gamma=A + 8 * act, residual_out=A + 12 * act,
             normed_out=A + 16 * act, normed_fp8=A + 20 * act, fp8_scale=A + 24 * act)
    p.update(over)
    return mfr.residual_add_rmsnorm_fp8_raw(p["x"], p["residual"], p["gamma"], eps,
                                            p["residual_out"], p["normed_out"], p["normed_fp8"],
                                            p["fp8_scale"], T_, H_, None)


def test_dense_fp8_validation():
    act = T * H * 2
    for name in ("x", "residual", "gamma", "residual_out", "normed_fp8", "fp8_scale"):
        assert dense_fp8_call(**{name: None}) == binding.MFR_ERR_NULL, name
    for name in ("x", "residual", "gamma", "residual_out", "normed_out"):
        assert dense_fp8_call(**{name: A + 30 * act + 8}) == binding.MFR_ERR_ALIGN, name
    assert dense_fp8_call(normed_fp8=A + 20 * act + 4) == binding.MFR_ERR_ALIGN
    assert dense_fp8_call(fp8_scale=A + 24 * act + 2) == binding.MFR_ERR_ALIGN
    for shape in ((-1, H), (T, 0), (T, 12), (T, 16392), (2**31, H)):
        assert dense_fp8_call(*shape) == binding.MFR_ERR_SHAPE, shape
    for eps in (-1.0, math.nan, math.inf):
        assert dense_fp8_call(eps=eps) == binding.MFR_ERR_SCALAR
    # codes on the residual output, the scale inside the codes, codes on an input,
    # the bf16 normed output on the codes
    assert dense_fp8_call(normed_fp8=A + 12 * act) == binding.MFR_ERR_ALIAS
    assert dense_fp8_call(fp8_scale=A + 20 * act + 64) == binding.MFR_ERR_ALIAS
    assert dense_fp8_call(normed_fp8=A) == binding.MFR_ERR_ALIAS
    assert dense_fp8_call(normed_out=A + 20 * act) == binding.MFR_ERR_ALIAS
    # without the optional bf16 output, its pointer is not examined
    assert dense_fp8_call(T_=0, normed_out=None) == binding.MFR_OK
    assert mfr.residual_add_rmsnorm_fp8_raw(None, None, None, 1e-6, None, None, None, None, 0, H,
                                            None) == binding.MFR_OK


def _path_in_subprocess(env_value, T, forced=0):
    """moe_finalize_rmsnorm_path(T, 6144, 8) in a fresh process whose
    environment holds MFR_PATH=env_value (read once, when the library loads)."""
    import subprocess
    import sys
    code = ("import ctypes, sys\n"
            "from top_finalize_residual_amd import build\n"
            "lib = ctypes.CDLL(build.LIB)\n"
            "lib.moe_finalize_rmsnorm_path.argtypes = [ctypes.c_int64] * 3\n"
            f"assert lib.mfr_tuning_force_launch({forced}, 0, 0) == 0\n"
            f"print(lib.moe_finalize_rmsnorm_path({T}, 6144, 8))\n")
    env = dict(os.environ)
    env.pop("MFR_PATH", None)
    if env_value is not None:
        env["MFR_PATH"] = env_value
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return int(r.stdout.strip()), r.stderr


def test_env_path_switch():
    """MFR_PATH sets the default path; an explicit override still wins; an
    unknown value is reported and ignored."""
    assert _path_in_subprocess(None, 8)[0] == mfr.PATH_TOKEN
    assert _path_in_subprocess(None, 8192)[0] == mfr.PATH_STREAM
    assert _path_in_subprocess("auto", 8192)[0] == mfr.PATH_STREAM
    assert _path_in_subprocess("stream", 8)[0] == mfr.PATH_STREAM
    assert _path_in_subprocess("token", 8192)[0] == mfr.PATH_TOKEN
    assert _path_in_subprocess("stream", 8, forced=mfr.PATH_TOKEN)[0] == mfr.PATH_TOKEN
    p, err = _path_in_subprocess("fastest", 8)
    assert p == mfr.PATH_TOKEN and "MFR_PATH=fastest" in err


def checked_call(R=T * K, bad_index=A + 71 * T * H * 2, T_=T, H_=H, K_=K, eps=1e-6, scale=2.5,
                 **over):
    p = _ptrs(**over)
    return binding.lib().moe_finalize_rmsnorm_checked(
        p["expert_out"], R, p["perm_idx"], p["topk_w"], p["shared_out"], p["residual"], p["gamma"],
        eps, scale, p["residual_out"], p["normed_out"], bad_index, T_, H_, K_, None)


def test_checked_validation():
    """moe_finalize_rmsnorm_checked: the plain op's checks plus R and the
    flag; with R known the overlap check covers all R rows of expert_out."""
    act = T * H * 2
    p = _ptrs()
    assert checked_call(R=-1) == binding.MFR_ERR_SHAPE
    assert checked_call(T_=T, H_=7) == binding.MFR_ERR_SHAPE
    assert checked_call(eps=math.nan) == binding.MFR_ERR_SCALAR
    assert checked_call(gamma=None) == binding.MFR_ERR_NULL
    assert checked_call(expert_out=None) == binding.MFR_ERR_NULL  # R > 0 needs the rows
    assert checked_call(bad_index=A + 71 * act + 2) == binding.MFR_ERR_ALIGN
    assert checked_call(bad_index=p["normed_out"] + 8) == binding.MFR_ERR_ALIAS
    assert checked_call(bad_index=p["perm_idx"]) == binding.MFR_ERR_ALIAS
    # an output inside expert_out's R rows, past the first 16 bytes that the
    # plain entry point (which is not told R) can check
    inside = p["expert_out"] + (T * K // 2) * H * 2
    assert checked_call(normed_out=inside) == binding.MFR_ERR_ALIAS
    assert checked_call(residual_out=inside) == binding.MFR_ERR_ALIAS
    # zero tokens: nothing examined, nothing launched
    assert binding.lib().moe_finalize_rmsnorm_checked(None, 0, None, None, None, None, None, 1e-6,
                                                      1.0, None, None, None, 0, H, K,
                                                      None) == binding.MFR_OK


def fp8_checked_call(T_=T, H_=H, K_=K, R=T * K, eps=1e-6, **over):
    act = T * H * 2
    p = dict(_ptrs(), normed_fp8=A + 80 * act, fp8_scale=A + 90 * act, bad_index=A + 91 * act)
    p.update(over)
    return mfr.moe_finalize_rmsnorm_fp8_checked_raw(
        p["expert_out"], R, p["perm_idx"], p["topk_w"], p["shared_out"], p["residual"], p["gamma"],
        eps, 2.5, p["residual_out"], p["normed_out"], p["normed_fp8"], p["fp8_scale"],
        p["bad_index"], T_, H_, K_, None)


def test_fp8_checked_validation():
    """moe_finalize_rmsnorm_fp8_checked: the FP8 call's checks plus R and the
    flag, with the overlap check over all R rows of expert_out."""
    act = T * H * 2
    p = dict(_ptrs(), normed_fp8=A + 80 * act, fp8_scale=A + 90 * act, bad_index=A + 91 * act)
    assert fp8_checked_call(R=-1) == binding.MFR_ERR_SHAPE
    assert fp8_checked_call(H_=12) == binding.MFR_ERR_SHAPE
    assert fp8_checked_call(eps=-1.0) == binding.MFR_ERR_SCALAR
    for name in ("perm_idx", "topk_w", "shared_out", "residual", "gamma", "residual_out",
                 "normed_fp8", "fp8_scale", "expert_out"):
        assert fp8_checked_call(**{name: None}) == binding.MFR_ERR_NULL, name
    assert fp8_checked_call(normed_fp8=p["normed_fp8"] + 4) == binding.MFR_ERR_ALIGN
    assert fp8_checked_call(bad_index=p["bad_index"] + 2) == binding.MFR_ERR_ALIGN
    assert fp8_checked_call(bad_index=p["fp8_scale"]) == binding.MFR_ERR_ALIAS
    assert fp8_checked_call(normed_fp8=p["expert_out"] + (T * K // 2) * H * 2) == \
        binding.MFR_ERR_ALIAS  # inside the R rows
    # the optional outputs are not examined when absent
    assert fp8_checked_call(normed_out=None, bad_index=None, T_=0) == binding.MFR_OK
    assert fp8_checked_call(R=0, expert_out=None, T_=0) == binding.MFR_OK


def test_launch_failure_is_reported_as_hip_error():
    """A call that passes every host check and then cannot be launched
    returns MFR_ERR_HIP, from every entry point. Without a GPU the HIP
    runtime refuses the launch itself; the fake addresses below are never
    dereferenced because nothing is enqueued. On a host with a GPU the
    launches would run, so the test is skipped there (the GPU tests cover
    real launches)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the calls would launch")
    p = _ptrs()
    lib = binding.lib()
    ins = (p["expert_out"], p["perm_idx"], p["topk_w"], p["shared_out"], p["residual"], p["gamma"])
    act = T * H * 2
    q, sc, flag = A + 80 * act, A + 90 * act, A + 91 * act
    calls = {
        "moe_finalize_rmsnorm": lambda: lib.moe_finalize_rmsnorm(
            *ins, 1e-6, 2.5, p["residual_out"], p["normed_out"], T, H, K, None),
        "moe_finalize_rmsnorm_checked": lambda: lib.moe_finalize_rmsnorm_checked(
            ins[0], T * K, *ins[1:], 1e-6, 2.5, p["residual_out"], p["normed_out"], flag, T, H, K,
            None),
        "moe_finalize_rmsnorm_fp8": lambda: lib.moe_finalize_rmsnorm_fp8(
            *ins, 1e-6, 2.5, p["residual_out"], p["normed_out"], q, sc, T, H, K, None),
        "moe_finalize_rmsnorm_fp8_checked": lambda: lib.moe_finalize_rmsnorm_fp8_checked(
            ins[0], T * K, *ins[1:], 1e-6, 2.5, p["residual_out"], None, q, sc, flag, T, H, K,
            None),
        "residual_add_rmsnorm": lambda: lib.residual_add_rmsnorm(
            p["shared_out"], p["residual"], p["gamma"], 1e-6, p["residual_out"], p["normed_out"],
            T, H, None),
        "residual_add_rmsnorm_fp8": lambda: lib.residual_add_rmsnorm_fp8(
            p["shared_out"], p["residual"], p["gamma"], 1e-6, p["residual_out"], None, q, sc, T, H,
            None),
    }
    for name, call in calls.items():
        assert call() == binding.MFR_ERR_HIP, name
    assert "HIP" in mfr.strerror(binding.MFR_ERR_HIP)
