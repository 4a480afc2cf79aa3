"""The deferred-finalize contract on the host: the producer's deferral check,
the MoEOutput containers and the torch custom-op registration (fake tensors,
no GPU)."""
import pytest
import torch

mfr = pytest.importorskip("top_finalize_residual_amd", reason="HIP library not built")


def test_defer_check_follows_the_kernel_limits():
    assert mfr.defer_moe_finalize(4, 6144, 8)
    assert mfr.defer_moe_finalize(8192, 6144, 8)
    assert mfr.defer_moe_finalize(1, 2048, 1)
    assert not mfr.defer_moe_finalize(4, 6143, 8)   # H not a multiple of 8
    assert not mfr.defer_moe_finalize(4, 32768, 8)  # H above 16384
    assert not mfr.defer_moe_finalize(4, 6144, 17)  # K above 16
    assert not mfr.defer_moe_finalize(-1, 6144, 8)


def test_moe_output_containers():
    E = torch.empty(32, 64, dtype=torch.bfloat16)
    p = torch.zeros(4, 8, dtype=torch.int32)
    w = torch.zeros(4, 8)
    u = mfr.UnfinalizedMoEOutput(E, p, w, scale=2.5)
    assert (u.num_tokens, u.hidden_size, u.top_k) == (4, 64, 8)
    assert mfr.MoEOutput(u, torch.empty(4, 64, dtype=torch.bfloat16)).deferred
    assert not mfr.MoEOutput(torch.empty(4, 64, dtype=torch.bfloat16),
                             torch.empty(4, 64, dtype=torch.bfloat16)).deferred


def test_custom_ops_are_registered_with_fake_kernels():
    from torch._subclasses.fake_tensor import FakeTensorMode
    assert hasattr(torch.ops.mfr, "moe_finalize_rmsnorm")
    assert hasattr(torch.ops.mfr, "residual_add_rmsnorm")
    assert hasattr(torch.ops.mfr, "moe_finalize_rmsnorm_")
    assert hasattr(torch.ops.mfr, "residual_add_rmsnorm_")
    with FakeTensorMode():
        x = torch.empty(4, 64, dtype=torch.bfloat16)
        r, n = mfr.fused_add_rmsnorm(x, torch.empty_like(x), torch.empty(64, dtype=torch.bfloat16),
                                     1e-6)
        assert r.shape == (4, 64) and n.shape == (4, 64)
        u = mfr.UnfinalizedMoEOutput(torch.empty(32, 64, dtype=torch.bfloat16),
                                     torch.zeros(4, 8, dtype=torch.int32), torch.zeros(4, 8))
        r, n = mfr.fused_add_rmsnorm(mfr.MoEOutput(u, x), x, torch.empty(64, dtype=torch.bfloat16),
                                     1e-6, in_place=True)
        assert r is x


def test_fp8_consumer_ops_with_fake_tensors():
    from torch._subclasses.fake_tensor import FakeTensorMode
    for name in ("moe_finalize_rmsnorm_fp8", "moe_finalize_rmsnorm_fp8_",
                 "residual_add_rmsnorm_fp8", "residual_add_rmsnorm_fp8_"):
        assert hasattr(torch.ops.mfr, name), name
    with FakeTensorMode():
        x = torch.empty(4, 64, dtype=torch.bfloat16)
        g = torch.empty(64, dtype=torch.bfloat16)
        r, q, sc = mfr.fused_add_rmsnorm(x, torch.empty_like(x), g, 1e-6, fp8=True)
        assert r.shape == (4, 64) and q.shape == (4, 64) and q.dtype == torch.float8_e4m3fn
        assert sc.shape == (4,) and sc.dtype == torch.float32
        u = mfr.UnfinalizedMoEOutput(torch.empty(32, 64, dtype=torch.bfloat16),
                                     torch.zeros(4, 8, dtype=torch.int32), torch.zeros(4, 8))
        res = torch.empty_like(x)
        out = mfr.fused_add_rmsnorm(mfr.MoEOutput(u, x), res, g, 1e-6, fp8=True, in_place=True)
        assert out[0] is res and len(out) == 3


def test_fp8_consumer_argument_rules():
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    g = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="not normed_out"):
        mfr.fused_add_rmsnorm(x, x.clone(), g, 1e-6, fp8=True, normed_out=torch.empty_like(x))
    with pytest.raises(ValueError, match="outputs of fp8=True"):
        mfr.fused_add_rmsnorm(x, x.clone(), g, 1e-6, fp8_scale=torch.empty(4))


def test_cpu_tensors_are_refused():
    # the product path has no CPU fallback
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        mfr.fused_add_rmsnorm(x, torch.zeros_like(x), torch.ones(64, dtype=torch.bfloat16), 1e-6)


OP_NAMES = ("moe_finalize_rmsnorm", "moe_finalize_rmsnorm_", "moe_finalize_rmsnorm_fp8",
            "moe_finalize_rmsnorm_fp8_", "residual_add_rmsnorm", "residual_add_rmsnorm_",
            "residual_add_rmsnorm_fp8", "residual_add_rmsnorm_fp8_")


def test_op_schemas_mark_what_each_op_writes():
    """The C++ definitions carry the alias annotations that tell torch which
    arguments each op writes (and that the in-place forms write the residual
    stream itself); no op returns anything."""
    written = {
        "moe_finalize_rmsnorm": ("residual_out", "normed_out"),
        "moe_finalize_rmsnorm_": ("residual", "normed_out"),
        "moe_finalize_rmsnorm_fp8": ("residual_out", "normed_fp8", "fp8_scale"),
        "moe_finalize_rmsnorm_fp8_": ("residual", "normed_fp8", "fp8_scale"),
        "residual_add_rmsnorm": ("residual_out", "normed_out"),
        "residual_add_rmsnorm_": ("residual", "normed_out"),
        "residual_add_rmsnorm_fp8": ("residual_out", "normed_fp8", "fp8_scale"),
        "residual_add_rmsnorm_fp8_": ("residual", "normed_fp8", "fp8_scale"),
    }
    for name in OP_NAMES:
        schema = getattr(torch.ops.mfr, name).default._schema
        assert len(schema.returns) == 0, name
        got = tuple(a.name for a in schema.arguments if a.alias_info is not None and
                    a.alias_info.is_write)
        assert got == written[name], (name, got)


def test_ops_refuse_cpu_tensors_directly():
    """Through torch.ops too, CPU tensors get a clear error, not a CPU result."""
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    g = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        torch.ops.mfr.residual_add_rmsnorm(x, x.clone(), g, 1e-6, torch.empty_like(x),
                                           torch.empty_like(x))
    u = (torch.zeros(32, 64, dtype=torch.bfloat16), torch.zeros(4, 8, dtype=torch.int32),
         torch.zeros(4, 8))
    with pytest.raises(ValueError, match="GPU"):
        torch.ops.mfr.moe_finalize_rmsnorm(*u, x, x.clone(), g, 1e-6, 1.0, torch.empty_like(x),
                                           torch.empty_like(x))
    with pytest.raises(TypeError, match="perm_idx"):
        torch.ops.mfr.moe_finalize_rmsnorm(u[0], u[1].long(), u[2], x, x.clone(), g, 1e-6, 1.0,
                                           torch.empty_like(x), torch.empty_like(x))
