"""GPU parity: the HIP library against the oracle, element by element, on the
seeded synthetic workloads, plus bit-exact checks of index handling, masked
slots, determinism, in-place use and graph replay."""
import numpy as np
import pytest
import torch

import synth
import top_finalize_residual_amd as mfr
from top_finalize_residual_amd import tuning
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

PATHS = [0, mfr.PATH_TOKEN, mfr.PATH_STREAM]
PATH_IDS = ["auto", "token", "stream"]

CONFIG_CASES = [(cfg, T) for cfg in ("tiny", "decode", "decode_masked", "batch512")
                for T in synth.CONFIGS[cfg]["Ts"]]


@pytest.fixture(scope="module")
def cfg_data():
    cache = {}

    def get(cfg, T):
        if (cfg, T) not in cache:
            d = synth.config_inputs(cfg, T)
            cache[(cfg, T)] = (d, gu.to_device(d), gu.oracle_for(d))
        return cache[(cfg, T)]
    return get


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("cfg,T", CONFIG_CASES, ids=[f"{c}-T{t}" for c, t in CONFIG_CASES])
def test_config_parity(cfg_data, cfg, T, path):
    d, dd, ref = cfg_data(cfg, T)
    r, n = gu.run(dd, d["eps"], d["scale"], path=path)
    gu.check(d, r, n, ref=ref)


@pytest.mark.parametrize("vpt", [1, 2, 3, 4])
@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
@pytest.mark.parametrize("cfg,T", [("tiny", 4), ("decode", 28), ("decode_masked", 64)])
def test_tile_variants(cfg_data, cfg, T, path, vpt):
    d, dd, ref = cfg_data(cfg, T)
    r, n = gu.run(dd, d["eps"], d["scale"], path=path, vpt=vpt)
    gu.check(d, r, n, ref=ref)


@pytest.mark.parametrize("store", [tuning.STORE_WRITE_BACK, tuning.STORE_WRITE_THROUGH],
                         ids=["write_back", "write_through"])
@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_store_policies(cfg_data, path, store):
    d, dd, ref = cfg_data("batch512", 512)
    r, n = gu.run(dd, d["eps"], d["scale"], path=path, store=store)
    gu.check(d, r, n, ref=ref)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_expert_sorted_layout(path):
    """The rows of expert_out grouped by expert, as a grouped GEMM2 writes
    them (the layout the bench also times), against the oracle; and the same
    tokens through the random layout give the same outputs bit for bit, since
    each token gathers the same values either way."""
    kw = dict(scale=2.5, weights="top8_of_256", seed=synth.seed_for("batch512", 512))
    d = synth.generate(512, 6144, 8, layout="expert_sorted", **kw)
    dr = synth.generate(512, 6144, 8, **kw)
    # same values per (token, slot): rearrange the random layout's rows into this one
    moved = dict(dr, expert_out=np.empty_like(dr["expert_out"]), perm_idx=d["perm_idx"])
    moved["expert_out"][d["perm_idx"].reshape(-1)] = dr["expert_out"][dr["perm_idx"].reshape(-1)]
    r, n = gu.run(gu.to_device(moved), d["eps"], d["scale"], path=path)
    gu.check(moved, r, n)
    r2, n2 = gu.run(gu.to_device(dr), d["eps"], d["scale"], path=path)
    assert np.array_equal(r, r2) and np.array_equal(n, n2)


def test_prefill_chunk_full_size():
    """The 8192-token prefill chunk at full size in the default (benchmarked)
    launch configuration: every token (8192 x 6144 elements of each output)
    against the oracle, which runs in threads over token ranges."""
    d = synth.config_inputs("prefill", 8192)
    assert mfr.moe_finalize_rmsnorm_path(8192, d["H"], d["K"]) == mfr.PATH_STREAM
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"])
    del dd
    gu.check_all_tokens(d, r, n)


RAGGED = [
    (1, 8, 1, 0.0), (3, 16, 2, 0.0), (5, 24, 3, 0.2), (7, 1000, 5, 0.1), (33, 2056, 9, 0.1),
    (17, 6152, 16, 0.05), (2, 16384, 16, 0.0), (300, 520, 4, 0.1), (257, 6144, 8, 0.0),
    (9, 12288, 7, 0.0), (65, 3072, 12, 0.0),
]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("T,H,K,mask", RAGGED, ids=[f"T{t}-H{h}-K{k}" for t, h, k, _ in RAGGED])
def test_ragged_shapes(T, H, K, mask, path):
    d = synth.generate(T, H, K, scale=2.5, mask_frac=mask, seed=1000 + T + H + K, extra_rows=3)
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"], path=path)
    gu.check(d, r, n)


def test_zero_tokens():
    d = synth.generate(0, 2048, 8, seed=5)
    dd = gu.to_device(d)
    r, n = mfr.moe_finalize_rmsnorm(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                    dd["shared_out"], dd["residual"], dd["gamma"], 1e-6, 1.0)
    assert r.shape == (0, 2048) and n.shape == (0, 2048)


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_masked_slots_never_read(path):
    """NaN in every row no valid index names, and NaN weights on masked slots:
    outputs bit-identical to the clean run."""
    d = synth.config_inputs("decode_masked", 64)
    dd = gu.to_device(d)
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=path)
    E = d["expert_out"].copy()
    used = np.zeros(d["R"], dtype=bool)
    used[d["perm_idx"][d["perm_idx"] >= 0]] = True
    E[~used] = 0x7FC0
    w = d["topk_w"].copy()
    w[d["perm_idx"] < 0] = np.nan
    dd2 = dict(dd, expert_out=gu.dev_bf16(E), topk_w=torch.from_numpy(w).cuda())
    r1, n1 = gu.run(dd2, d["eps"], d["scale"], path=path)
    assert np.array_equal(r0, r1) and np.array_equal(n0, n1)


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_masked_slot_position_is_irrelevant(path):
    """Moving a token's masked slots to the end leaves its outputs bit-identical."""
    d = synth.config_inputs("decode_masked", 64)
    dd = gu.to_device(d)
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=path)
    p, w = d["perm_idx"].copy(), d["topk_w"].copy()
    order = np.argsort(p < 0, axis=1, kind="stable")  # valid slots first, in their order
    p2, w2 = np.take_along_axis(p, order, 1), np.take_along_axis(w, order, 1)
    assert not np.array_equal(p2, p)
    dd2 = dict(dd, perm_idx=torch.from_numpy(p2).cuda(), topk_w=torch.from_numpy(w2).cuda())
    r1, n1 = gu.run(dd2, d["eps"], d["scale"], path=path)
    assert np.array_equal(r0, r1) and np.array_equal(n0, n1)


@pytest.mark.parametrize("variant", ["all_masked", "zero_weights"])
@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_no_routed_contribution(path, variant):
    """With every slot masked, or every weight zero, residual_out is the
    rounded shared + residual: bit-exact with the oracle wherever that fp32 sum
    is exact."""
    d = synth.generate(16, 2048, 8, scale=2.5, seed=77)
    if variant == "all_masked":
        d["perm_idx"][:] = -1
    else:
        d["topk_w"][:] = 0.0
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"], path=path)
    ref = gu.check(d, r, n)
    sh, rs = gu.bf16_f64(d["shared_out"]), gu.bf16_f64(d["residual"])
    exact32 = (sh + rs).astype(np.float32).astype(np.float64) == sh + rs
    assert exact32.mean() > 0.9
    assert np.array_equal(r[exact32], ref["residual_out"][exact32])


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_permutation_handling_bitexact(path):
    """Gathering through a permutation equals, bit for bit, reading rows that
    were pre-permuted on the host through the identity map."""
    d = synth.config_inputs("decode", 64)
    dd = gu.to_device(d)
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=path)
    T, K = d["perm_idx"].shape
    E2 = d["expert_out"][d["perm_idx"].reshape(-1)]
    ident = np.arange(T * K, dtype=np.int32).reshape(T, K)
    dd2 = dict(dd, expert_out=gu.dev_bf16(E2), perm_idx=torch.from_numpy(ident).cuda())
    r1, n1 = gu.run(dd2, d["eps"], d["scale"], path=path)
    assert np.array_equal(r0, r1) and np.array_equal(n0, n1)


def test_deterministic_and_path_independent():
    d = synth.config_inputs("batch512", 512)
    dd = gu.to_device(d)
    ra, na = gu.run(dd, d["eps"], d["scale"], path=mfr.PATH_STREAM)
    rb, nb = gu.run(dd, d["eps"], d["scale"], path=mfr.PATH_STREAM)
    assert np.array_equal(ra, rb) and np.array_equal(na, nb)
    rt, nt = gu.run(dd, d["eps"], d["scale"], path=mfr.PATH_TOKEN)
    # the sum s is formed the same way in every layout: residual_out is identical
    assert np.array_equal(ra, rt)
    # normed_out depends on the reduction tree of the layout; both pass the gate
    gu.check(d, rt, nt)
    for vpt in (1, 2, 4):
        rv, _ = gu.run(dd, d["eps"], d["scale"], path=mfr.PATH_TOKEN, vpt=vpt)
        assert np.array_equal(ra, rv), vpt
    # the store policy changes only where the bytes go, never their value
    for store in (tuning.STORE_WRITE_BACK, tuning.STORE_WRITE_THROUGH):
        rs, ns = gu.run(dd, d["eps"], d["scale"], path=mfr.PATH_STREAM, store=store)
        assert np.array_equal(ra, rs) and np.array_equal(na, ns), store


def test_batch_invariance():
    """A token's outputs do not depend on the other tokens in the call."""
    d = synth.config_inputs("decode", 64)
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"], path=mfr.PATH_TOKEN)
    for t in (0, 17, 63):
        one = {k: (v[t:t + 1].contiguous() if k in ("perm_idx", "topk_w", "shared_out", "residual")
                   else v) for k, v in dd.items()}
        r1, n1 = gu.run(one, d["eps"], d["scale"], path=mfr.PATH_TOKEN)
        assert np.array_equal(r1[0], r[t]) and np.array_equal(n1[0], n[t])


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_in_place_residual(path):
    d = synth.config_inputs("decode", 28)
    dd = gu.to_device(d)
    r0, n0 = gu.run(dd, d["eps"], d["scale"], path=path)
    resid = dd["residual"].clone()
    dd2 = dict(dd, residual=resid)
    r1, n1 = gu.run(dd2, d["eps"], d["scale"], path=path, residual_out=resid)
    assert np.array_equal(r0, r1) and np.array_equal(n0, n1)
    assert np.array_equal(gu.host_u16(resid), r0)


def test_graph_capture_replay():
    """Calls captured into a HIP graph (through torch) replay correctly, again
    and again, with eager work and synchronisations between replays."""
    d = synth.config_inputs("decode", 28)
    dd = gu.to_device(d)
    r_eager, n_eager = gu.run(dd, d["eps"], d["scale"])
    r_out = torch.empty_like(dd["residual"])
    n_out = torch.empty_like(dd["residual"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):  # warm up on the capture stream
            mfr.moe_finalize_rmsnorm(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                     dd["shared_out"], dd["residual"], dd["gamma"], d["eps"],
                                     d["scale"], residual_out=r_out, normed_out=n_out)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(4):
            mfr.moe_finalize_rmsnorm(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                     dd["shared_out"], dd["residual"], dd["gamma"], d["eps"],
                                     d["scale"], residual_out=r_out, normed_out=n_out)
    for i in range(20):
        r_out.fill_(0)
        n_out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gu.host_u16(r_out), r_eager), i
        assert np.array_equal(gu.host_u16(n_out), n_eager), i


def test_graph_back_to_back_in_place_chain():
    """1000 graph replays launched back to back with no synchronisation,
    each updating the residual stream in place, so that every replay reads
    what the previous one wrote. The final state must equal, bit for bit,
    1000 eager calls: nothing carries over between launches except the
    data, and no launch may start before the previous one finished."""
    d = synth.config_inputs("decode", 4)
    dd = gu.to_device(d)
    n_out = torch.empty_like(dd["residual"])

    def step(res):
        mfr.moe_finalize_rmsnorm(dd["expert_out"], dd["perm_idx"], dd["topk_w"],
                                 dd["shared_out"], res, dd["gamma"], d["eps"], d["scale"],
                                 residual_out=res, normed_out=n_out)
    eager = dd["residual"].clone()
    for _ in range(1000):
        step(eager)
    torch.cuda.synchronize()
    want_res, want_n = gu.host_u16(eager), gu.host_u16(n_out)

    chained = dd["residual"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(chained.clone())  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(chained)
    torch.cuda.synchronize()
    chained.copy_(dd["residual"])
    n_out.fill_(0)
    torch.cuda.synchronize()
    for _ in range(1000):
        g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_u16(chained), want_res)
    assert np.array_equal(gu.host_u16(n_out), want_n)
    assert not np.array_equal(want_res, gu.host_u16(dd["residual"]))


def test_row_offsets_beyond_2gib():
    """expert_out larger than 2^31 bytes: rows past that mark are gathered with
    64-bit row offsets. Only the referenced rows are filled; the others are
    never read."""
    T, H, K = 64, 6144, 8
    row_bytes = H * 2
    R = (2**31 // row_bytes) + 4096  # ~2.2 GB of rows
    d = synth.generate(T, H, K, scale=2.5, seed=321)
    rng = np.random.default_rng(9)
    hi = R - 1 - rng.choice(4000, size=T * K, replace=False)  # rows above 2^31 bytes
    assert hi.min() * row_bytes >= 2**31
    perm_hi = hi.astype(np.int32).reshape(T, K)
    E = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
    rows_dev = gu.dev_bf16(d["expert_out"])  # [T*K, H], row j goes to hi[j]
    E[torch.from_numpy(hi).cuda()] = rows_dev
    dd = gu.to_device(d)
    dd["expert_out"] = E
    dd["perm_idx"] = torch.from_numpy(perm_hi).cuda()
    r, n = gu.run(dd, d["eps"], d["scale"])
    # the oracle sees the same rows at compact indices
    d_ref = dict(d, perm_idx=np.arange(T * K, dtype=np.int32).reshape(T, K))
    gu.check(d_ref, r, n)
    del E
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", [mfr.PATH_TOKEN, mfr.PATH_STREAM], ids=["token", "stream"])
def test_special_values_propagate(path):
    """Inf and NaN inputs follow the definition on both sides. A token with
    one infinite residual element gets Inf in residual_out there; its sum of
    squares is infinite, so that element normalises to NaN (inf/inf) and the
    others to +-0. A token with one NaN shared element gets NaN there in
    residual_out, and its whole normed row is NaN. Other tokens are
    untouched: special positions are compared exactly, finite values
    through the gate."""
    d = synth.generate(3, 2048, 8, scale=2.5, seed=31)
    d["residual"] = d["residual"].copy()
    d["shared_out"] = d["shared_out"].copy()
    d["residual"][1, 5] = 0x7F80      # +inf
    d["shared_out"][2, 7] = 0x7FC0    # NaN
    dd = gu.to_device(d)
    r, n = gu.run(dd, d["eps"], d["scale"], path=path)
    ref = gu.oracle_for(d)
    for got, want_exact, what in ((r, ref["s"], "residual_out"), (n, ref["normed_exact"], "normed_out")):
        g = gu.bf16_f64(got)
        assert np.array_equal(np.isnan(g), np.isnan(want_exact)), what
        assert np.array_equal(np.isinf(g), np.isinf(want_exact)), what
        assert np.array_equal(np.sign(g[np.isinf(g)]), np.sign(want_exact[np.isinf(want_exact)])), what
        fin = np.isfinite(want_exact)
        assert np.all(np.abs(g[fin] - want_exact[fin]) <= gu.REL * np.abs(want_exact[fin]) + gu.ABS), what
    g_r, g_n = gu.bf16_f64(r), gu.bf16_f64(n)
    assert np.isinf(g_r[1, 5]) and np.isnan(g_n[1, 5])
    assert np.all(g_n[1, np.arange(2048) != 5] == 0.0)
    assert np.isnan(g_r[2, 7]) and np.all(np.isnan(g_n[2]))
    assert np.all(np.isfinite(g_r[0])) and np.all(np.isfinite(g_n[0]))


def test_eps_zero_zero_row_is_nan():
    """eps = 0 and a token whose sum is exactly zero: 0/0 gives NaN in the
    normed output on both sides; residual_out is +-0."""
    d = synth.generate(2, 256, 2, scale=1.0, seed=8)
    d["topk_w"][0] = 0.0
    d["residual"][0] = d["shared_out"][0] ^ np.uint16(0x8000)  # residual = -shared
    dd = gu.to_device(d)
    r, n = gu.run(dd, 0.0, 1.0)
    ref = gu.oracle_for(dict(d, eps=0.0))
    assert np.all(gu.bf16_f64(r[0]) == 0)
    assert np.all(np.isnan(gu.bf16_f64(n[0]))) and np.all(np.isnan(ref["normed_exact"][0]))
    gu.check(dict(d, eps=0.0), r[1:], n[1:], ref={k: v[1:] for k, v in ref.items()})
