"""GPU robustness: concurrent callers on separate streams, argument errors
raised through the binding, and zero-token calls of every entry point."""
import threading

import numpy as np
import pytest
import torch

import synth
import top_finalize_residual_amd as mfr
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_concurrent_threads_and_streams():
    """Four host threads, each with its own stream and inputs, launch
    repeatedly at the same time; every result equals its single-threaded one."""
    cases = [synth.generate(T, 2048 if i % 2 else 6144, 8, scale=2.5, seed=900 + i)
             for i, T in enumerate((1, 28, 64, 512))]
    devs = [gu.to_device(d) for d in cases]
    want = [gu.run(dd, d["eps"], d["scale"]) for d, dd in zip(cases, devs)]
    outs = [None] * len(cases)
    errors = []

    def worker(i):
        try:
            d, dd = cases[i], devs[i]
            s = torch.cuda.Stream()
            r = torch.empty_like(dd["residual"])
            n = torch.empty_like(dd["residual"])
            with torch.cuda.stream(s):
                for _ in range(50):
                    mfr.moe_finalize_rmsnorm(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                             dd["shared_out"], dd["residual"], dd["gamma"],
                                             d["eps"], d["scale"], residual_out=r, normed_out=n)
            s.synchronize()
            outs[i] = (gu.host_u16(r), gu.host_u16(n))
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (r0, n0), (r1, n1) in zip(want, outs):
        assert np.array_equal(r0, r1) and np.array_equal(n0, n1)


def test_binding_rejects_bad_tensors_before_launch():
    d = synth.generate(4, 2048, 8, seed=901)
    dd = gu.to_device(d)
    args = [dd[k] for k in ("expert_out", "perm_idx", "topk_w", "shared_out", "residual", "gamma")]
    # a bf16 view one element in: 2-byte aligned, refused by the library
    big = torch.empty(4 * 2048 + 8, dtype=torch.bfloat16, device="cuda")
    shifted = big[1:1 + 4 * 2048].view(4, 2048)
    with pytest.raises(mfr.MFRError) as e:
        mfr.moe_finalize_rmsnorm(*args, d["eps"], d["scale"], residual_out=shifted)
    assert e.value.status == 3  # MFR_ERR_ALIGN
    # outputs overlapping an input
    with pytest.raises(mfr.MFRError) as e:
        mfr.moe_finalize_rmsnorm(*args, d["eps"], d["scale"], normed_out=dd["shared_out"])
    assert e.value.status == 4  # MFR_ERR_ALIAS
    # wrong dtype / layout / device are refused by the binding itself
    with pytest.raises(TypeError):
        mfr.moe_finalize_rmsnorm(args[0].float(), *args[1:], d["eps"], d["scale"])
    strided = torch.empty(2048, 4, dtype=torch.bfloat16, device="cuda").t()  # [4, 2048], not contiguous
    with pytest.raises(ValueError):
        mfr.moe_finalize_rmsnorm(*args[:3], strided, *args[4:], d["eps"], d["scale"])
    with pytest.raises(ValueError):
        mfr.moe_finalize_rmsnorm(*args, d["eps"], d["scale"],
                                 residual_out=torch.empty(4, 2048, dtype=torch.bfloat16))
    # FP8 outputs of the wrong length are refused before anything is written
    with pytest.raises(ValueError, match="fp8_scale"):
        mfr.moe_finalize_rmsnorm_fp8(*args, d["eps"], d["scale"],
                                     fp8_scale=torch.empty(3, device="cuda"))
    with pytest.raises(ValueError, match="normed_out"):
        mfr.moe_finalize_rmsnorm_fp8(*args, d["eps"], d["scale"],
                                     normed_out=torch.empty(3, 2048, dtype=torch.bfloat16,
                                                            device="cuda"))
    # a masked-everything call with NaN weights still works (weights of masked slots ignored)
    p = torch.full_like(dd["perm_idx"], -1)
    w = torch.full_like(dd["topk_w"], float("nan"))
    r, n = mfr.moe_finalize_rmsnorm(args[0], p, w, *args[3:], d["eps"], d["scale"])
    torch.cuda.synchronize()
    assert not torch.isnan(r.float()).any() and not torch.isnan(n.float()).any()


def test_zero_tokens_every_entry_point():
    d = synth.generate(0, 2048, 8, seed=902)
    dd = gu.to_device(d)
    r, q, sc, n = mfr.moe_finalize_rmsnorm_fp8(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                               dd["shared_out"], dd["residual"], dd["gamma"],
                                               1e-6, 1.0, bf16_normed=True)
    assert q.shape == (0, 2048) and sc.shape == (0,) and n.shape == (0, 2048)
    r, n = mfr.residual_add_rmsnorm(dd["shared_out"], dd["residual"], dd["gamma"], 1e-6)
    assert r.shape == (0, 2048)


def test_env_log_reports_each_launch():
    """MFR_LOG=1 prints the launch shape the host chose for every call."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import torch, synth\n"
            "import top_finalize_residual_amd as mfr\n"
            "from tests import gpu_util as gu\n"
            "for T in (4, 1024):\n"
            "    d = synth.generate(T, 2048, 8, seed=5)\n"
            "    gu.run(gu.to_device(d), d['eps'], d['scale'])\n"
            "torch.cuda.synchronize()\n")
    env = dict(os.environ, MFR_LOG="1")
    env.pop("MFR_PATH", None)
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("moe_finalize_rmsnorm: T=")]
    assert len(lines) == 2, r.stderr[-2000:]
    assert "T=4 H=2048 K=8 variant=top8 out=bf16 path=token" in lines[0]
    assert "T=1024 H=2048 K=8 variant=top8 out=bf16 path=stream" in lines[1]


def test_env_log_store_policy_follows_the_output_bytes():
    """The automatic output stores: write-through on the token path up to 64
    tokens with bf16 output and write-back above (T = 64 and 65) or with FP8
    output (T = 28), the dense tail alike (T = 28, bf16 and FP8 output),
    write-back on the stream
    path while both outputs together stay within 12 MiB and write-through
    above that (T = 512 and 513 at H = 6144, 1536 and 1537 at H = 2048). Read
    from the launch log of a child process."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import torch, synth\n"
            "from tests import gpu_util as gu\n"
            "for T, H in ((64, 6144), (65, 6144), (511, 6144), (512, 6144), (513, 6144),\n"
            "             (1536, 2048), (1537, 2048)):\n"
            "    d = synth.generate(T, H, 8, seed=6)\n"
            "    gu.run(gu.to_device(d), d['eps'], d['scale'])\n"
            "from tests.test_fp8_gpu import run_fp8\n"
            "d = synth.generate(28, 6144, 8, seed=6)\n"
            "run_fp8(gu.to_device(d), d)\n"
            "from tests.test_dense_gpu import run_dense, run_dense_fp8\n"
            "d = synth.dense_inputs(28, 6144, seed=6)\n"
            "run_dense(d)\n"
            "run_dense_fp8(d, bf16_normed=False)\n"
            "torch.cuda.synchronize()\n")
    env = dict(os.environ, MFR_LOG="1")
    env.pop("MFR_PATH", None)
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("moe_finalize_rmsnorm: T=")]
    assert len(lines) == 10, r.stderr[-2000:]
    want = (("T=64 H=6144", "path=token", "stores=write-through"),
            ("T=65 H=6144", "path=token", "stores=write-back"),
            ("T=511 H=6144", "path=token", "stores=write-back"),
            ("T=512 H=6144", "path=stream", "stores=write-back"),
            ("T=513 H=6144", "path=stream", "stores=write-through"),
            ("T=1536 H=2048", "path=stream", "stores=write-back"),
            ("T=1537 H=2048", "path=stream", "stores=write-through"),
            ("T=28 H=6144", "out=fp8 path=token", "stores=write-back"),
            ("T=28 H=6144", "variant=dense out=bf16 path=token", "stores=write-through"),
            ("T=28 H=6144", "variant=dense out=fp8 path=token", "stores=write-back"))
    for ln, parts in zip(lines, want):
        for part in parts:
            assert part in ln, (part, ln)
