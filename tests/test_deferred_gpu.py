"""GPU checks of the deferred-finalize contract: the consumer norm dispatches
to the right kernel, bit-identical to the direct calls, and a captured graph of
a decoder tail replays correctly."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_finalize_residual_amd as mfr
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _dev(d):
    dd = gu.to_device(d)
    return dd, mfr.UnfinalizedMoEOutput(dd["expert_out"], dd["perm_idx"], dd["topk_w"], d["scale"])


@pytest.mark.parametrize("T", [4, 28, 512])
def test_deferred_moe_output_equals_direct_call(T):
    d = synth.generate(T, 6144, 8, scale=2.5, mask_frac=0.05, seed=600 + T)
    dd, u = _dev(d)
    assert mfr.defer_moe_finalize(T, 6144, 8)
    r, n = mfr.fused_add_rmsnorm(mfr.MoEOutput(u, dd["shared_out"]), dd["residual"], dd["gamma"],
                                 d["eps"])
    torch.cuda.synchronize()
    r0, n0 = gu.run(dd, d["eps"], d["scale"])
    assert np.array_equal(gu.host_u16(r), r0) and np.array_equal(gu.host_u16(n), n0)


def test_finalized_routed_part_goes_through_the_fused_kernel():
    """A MoEOutput whose routed part is already a [T, H] tensor: routed +
    shared + residual with one rounding, then RMSNorm (checked against the
    oracle with K = 1, identity map, weight 1)."""
    d = synth.generate(64, 2048, 1, scale=1.0, seed=61)
    routed = d["expert_out"][d["perm_idx"][:, 0]]  # one [T, H] routed tensor
    dd = gu.to_device(d)
    r, n = mfr.fused_add_rmsnorm(mfr.MoEOutput(gu.dev_bf16(routed), dd["shared_out"]),
                                 dd["residual"], dd["gamma"], d["eps"])
    torch.cuda.synchronize()
    ident = np.arange(64, dtype=np.int32)[:, None]
    ref = oracle.finalize_rmsnorm(routed, ident, np.ones((64, 1), np.float32), d["shared_out"],
                                  d["residual"], d["gamma"], d["eps"], 1.0)
    gu.check(d, gu.host_u16(r), gu.host_u16(n), ref=ref)


def test_plain_tensor_goes_to_the_dense_kernel_in_place():
    d = synth.dense_inputs(28, 6144, seed=62)
    x, res, g = gu.dev_bf16(d["x"]), gu.dev_bf16(d["residual"]), gu.dev_bf16(d["gamma"])
    r0, n0 = mfr.residual_add_rmsnorm(x, res, g, d["eps"])
    r, n = mfr.fused_add_rmsnorm(x, res, g, d["eps"], in_place=True)
    torch.cuda.synchronize()
    assert r.data_ptr() == res.data_ptr()
    assert np.array_equal(gu.host_u16(r), gu.host_u16(r0))
    assert np.array_equal(gu.host_u16(n), gu.host_u16(n0))


def test_custom_ops_pass_opcheck():
    d = synth.generate(4, 2048, 8, seed=63)
    dd = gu.to_device(d)
    ro, no = torch.empty_like(dd["residual"]), torch.empty_like(dd["residual"])
    torch.library.opcheck(torch.ops.mfr.moe_finalize_rmsnorm.default,
                          (dd["expert_out"], dd["perm_idx"], dd["topk_w"], dd["shared_out"],
                           dd["residual"], dd["gamma"], d["eps"], d["scale"], ro, no),
                          test_utils=("test_schema", "test_faketensor"))
    torch.library.opcheck(torch.ops.mfr.residual_add_rmsnorm.default,
                          (dd["shared_out"], dd["residual"], dd["gamma"], d["eps"], ro, no),
                          test_utils=("test_schema", "test_faketensor"))
    # the in-place forms: the residual stream is the one mutated argument
    torch.library.opcheck(torch.ops.mfr.moe_finalize_rmsnorm_.default,
                          (dd["expert_out"], dd["perm_idx"], dd["topk_w"], dd["shared_out"],
                           dd["residual"].clone(), dd["gamma"], d["eps"], d["scale"], no),
                          test_utils=("test_schema", "test_faketensor"))
    torch.library.opcheck(torch.ops.mfr.residual_add_rmsnorm_.default,
                          (dd["shared_out"], dd["residual"].clone(), dd["gamma"], d["eps"], no),
                          test_utils=("test_schema", "test_faketensor"))


@pytest.mark.parametrize("deferred", [True, False], ids=["moe", "dense"])
def test_in_place_forms_equal_out_of_place(deferred):
    """in_place=True and residual_out=residual both update the residual
    stream through the in-place op, bit-identical to the out-of-place op."""
    d = synth.generate(28, 6144, 8, scale=2.5, seed=67)
    dd, u = _dev(d)
    hidden = mfr.MoEOutput(u, dd["shared_out"]) if deferred else dd["shared_out"]
    r0, n0 = mfr.fused_add_rmsnorm(hidden, dd["residual"], dd["gamma"], d["eps"])
    for kw in ({"in_place": True}, {"residual_out": "self"}):
        res = dd["residual"].clone()
        if kw.get("residual_out") == "self":
            kw = {"residual_out": res}
        r, n = mfr.fused_add_rmsnorm(hidden, res, dd["gamma"], d["eps"], **kw)
        torch.cuda.synchronize()
        assert r is res
        assert torch.equal(r.view(torch.int16), r0.view(torch.int16))
        assert torch.equal(n.view(torch.int16), n0.view(torch.int16))
    with pytest.raises(ValueError, match="in_place"):
        mfr.fused_add_rmsnorm(hidden, dd["residual"], dd["gamma"], d["eps"], in_place=True,
                              residual_out=torch.empty_like(dd["residual"]))


def test_decoder_tail_graph_replay():
    """Two layer boundaries of a decode step: a dense (attention) output into
    the post-attention norm, then the MoE layer's deferred output into the next
    layer's input norm; captured once, replayed many times."""
    T, H, K = 28, 6144, 8
    d = synth.generate(T, H, K, scale=2.5, seed=64)
    dd, u = _dev(d)
    attn_out = gu.dev_bf16(synth.dense_inputs(T, H, seed=65)["x"])
    res0 = dd["residual"].clone()
    g1, g2 = dd["gamma"], gu.dev_bf16(synth.dense_inputs(T, H, seed=66)["gamma"])

    def step(res):
        res, h = mfr.fused_add_rmsnorm(attn_out, res, g1, d["eps"], in_place=True)
        res, h2 = mfr.fused_add_rmsnorm(mfr.MoEOutput(u, dd["shared_out"]), res, g2, d["eps"],
                                        in_place=True, normed_out=h)
        return res, h2

    res_e = res0.clone()
    _, h_e = step(res_e)
    torch.cuda.synchronize()
    want_res, want_h = gu.host_u16(res_e), gu.host_u16(h_e)

    res_g = res0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(res_g.clone())
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _, h_g = step(res_g)
    for i in range(10):
        res_g.copy_(res0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gu.host_u16(res_g), want_res), i
        assert np.array_equal(gu.host_u16(h_g), want_h), i


def test_decoder_tail_graph_replay_fp8():
    """The same two boundaries with FP8 outputs, as in a model whose
    projections run in FP8: the post-attention norm and the next layer's input
    norm both write E4M3 codes and per-token scales. Captured once, replayed
    many times, every replay bit-identical to eager."""
    T, H, K = 28, 6144, 8
    d = synth.generate(T, H, K, scale=2.5, seed=74)
    dd, u = _dev(d)
    attn_out = gu.dev_bf16(synth.dense_inputs(T, H, seed=75)["x"])
    res0 = dd["residual"].clone()
    g1, g2 = dd["gamma"], gu.dev_bf16(synth.dense_inputs(T, H, seed=76)["gamma"])
    outs = [(torch.empty((T, H), dtype=torch.float8_e4m3fn, device="cuda"),
             torch.empty((T,), dtype=torch.float32, device="cuda")) for _ in range(2)]

    def step(res):
        mfr.fused_add_rmsnorm(attn_out, res, g1, d["eps"], in_place=True, fp8=True,
                              normed_fp8=outs[0][0], fp8_scale=outs[0][1])
        mfr.fused_add_rmsnorm(mfr.MoEOutput(u, dd["shared_out"]), res, g2, d["eps"],
                              in_place=True, fp8=True, normed_fp8=outs[1][0],
                              fp8_scale=outs[1][1])

    def snapshot(res):
        return [res.view(torch.int16).clone()] + [t.view(torch.uint8).clone() for q, sc in outs
                                                   for t in (q, sc.view(torch.uint8))]
    res_e = res0.clone()
    step(res_e)
    torch.cuda.synchronize()
    want = snapshot(res_e)

    res_g = res0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(res_g.clone())
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(res_g)
    for i in range(10):
        res_g.copy_(res0)
        for q, sc in outs:
            q.view(torch.uint8).zero_()
            sc.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(res_g)
        assert all(torch.equal(a, b) for a, b in zip(got, want)), i


@pytest.mark.parametrize("in_place", [False, True], ids=["separate", "in_place"])
@pytest.mark.parametrize("deferred", [True, False], ids=["moe", "dense"])
def test_fp8_consumer_equals_direct_calls(deferred, in_place):
    """fused_add_rmsnorm(fp8=True): the residual stream, codes and scales
    bit-identical to the direct FP8 calls, for a deferred MoEOutput (fused
    kernel) and a plain tensor (dense kernel), in place or not."""
    d = synth.generate(28, 6144, 8, scale=2.5, mask_frac=0.05, seed=68)
    dd, u = _dev(d)
    if deferred:
        hidden = mfr.MoEOutput(u, dd["shared_out"])
        r0, q0, s0, _ = mfr.moe_finalize_rmsnorm_fp8(dd["expert_out"], dd["perm_idx"],
                                                     dd["topk_w"], dd["shared_out"],
                                                     dd["residual"], dd["gamma"], d["eps"],
                                                     d["scale"])
    else:
        hidden = dd["shared_out"]
        r0, q0, s0, _ = mfr.residual_add_rmsnorm_fp8(dd["shared_out"], dd["residual"],
                                                     dd["gamma"], d["eps"])
    res = dd["residual"].clone()
    r, q, s = mfr.fused_add_rmsnorm(hidden, res, dd["gamma"], d["eps"], fp8=True,
                                    in_place=in_place)
    torch.cuda.synchronize()
    assert (r is res) == in_place
    assert q.dtype == torch.float8_e4m3fn and s.shape == (28,)
    assert torch.equal(r.view(torch.int16), r0.view(torch.int16))
    assert torch.equal(q.view(torch.uint8), q0.view(torch.uint8))
    assert torch.equal(s.view(torch.int32), s0.view(torch.int32))


def test_fp8_custom_ops_pass_opcheck():
    d = synth.generate(4, 2048, 8, seed=69)
    dd = gu.to_device(d)
    ro = torch.empty_like(dd["residual"])
    # the codes as uint8 (the ops take either): opcheck's schema check compares
    # tensor values with arithmetic that torch does not provide for float8
    q = torch.empty(dd["residual"].shape, dtype=torch.uint8, device="cuda")
    s = torch.empty((4,), dtype=torch.float32, device="cuda")
    routed = (dd["expert_out"], dd["perm_idx"], dd["topk_w"], dd["shared_out"])
    utils = ("test_schema", "test_faketensor")
    torch.library.opcheck(torch.ops.mfr.moe_finalize_rmsnorm_fp8.default,
                          routed + (dd["residual"], dd["gamma"], d["eps"], d["scale"], ro, q, s),
                          test_utils=utils)
    torch.library.opcheck(torch.ops.mfr.moe_finalize_rmsnorm_fp8_.default,
                          routed + (dd["residual"].clone(), dd["gamma"], d["eps"], d["scale"], q, s),
                          test_utils=utils)
    torch.library.opcheck(torch.ops.mfr.residual_add_rmsnorm_fp8.default,
                          (dd["shared_out"], dd["residual"], dd["gamma"], d["eps"], ro, q, s),
                          test_utils=utils)
    torch.library.opcheck(torch.ops.mfr.residual_add_rmsnorm_fp8_.default,
                          (dd["shared_out"], dd["residual"].clone(), dd["gamma"], d["eps"], q, s),
                          test_utils=utils)


def test_ops_pass_every_opcheck():
    """All of torch.library.opcheck's default checks (schema, autograd
    registration, fake tensors, AOT dispatch with dynamic shapes) on the C++
    operators, out of place and in place."""
    d = synth.generate(4, 2048, 8, seed=64)
    dd = gu.to_device(d)
    ro, no = torch.empty_like(dd["residual"]), torch.empty_like(dd["residual"])
    T, H = dd["residual"].shape
    # codes as uint8, as in the FP8 opcheck above: the schema check compares
    # values with arithmetic torch lacks for float8
    q = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    sc = torch.empty((T,), dtype=torch.float32, device="cuda")
    moe = (dd["expert_out"], dd["perm_idx"], dd["topk_w"], dd["shared_out"])
    cases = [
        ("moe_finalize_rmsnorm", (*moe, dd["residual"], dd["gamma"], d["eps"], d["scale"], ro, no)),
        ("moe_finalize_rmsnorm_", (*moe, dd["residual"].clone(), dd["gamma"], d["eps"], d["scale"],
                                   no)),
        ("moe_finalize_rmsnorm_fp8", (*moe, dd["residual"], dd["gamma"], d["eps"], d["scale"], ro,
                                      q, sc)),
        ("residual_add_rmsnorm", (dd["shared_out"], dd["residual"], dd["gamma"], d["eps"], ro, no)),
        ("residual_add_rmsnorm_fp8_", (dd["shared_out"], dd["residual"].clone(), dd["gamma"],
                                       d["eps"], q, sc)),
    ]
    for name, args in cases:
        torch.library.opcheck(getattr(torch.ops.mfr, name).default, args)


def test_ops_empty_call_and_library_errors():
    """Through torch.ops: T = 0 enqueues nothing and succeeds; an output that
    overlaps an input is refused by the library, whose status text the
    error carries."""
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    torch.ops.mfr.residual_add_rmsnorm(x, x.clone(), g, 1e-6, x.clone(), x.clone())
    torch.ops.mfr.moe_finalize_rmsnorm(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"),
                                       torch.zeros((0, 8), dtype=torch.int32, device="cuda"),
                                       torch.zeros((0, 8), device="cuda"), x, x.clone(), g, 1e-6,
                                       1.0, x.clone(), x.clone())
    torch.cuda.synchronize()
    a = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros_like(a)
    with pytest.raises(RuntimeError, match="overlaps"):
        torch.ops.mfr.residual_add_rmsnorm(a, r, g, 1e-6, a, torch.empty_like(a))
