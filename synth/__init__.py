"""Seeded synthetic inputs for the fused MoE finalize + RMSNorm.

Both sides of every parity check draw their inputs from here: the oracle and
the GPU library receive the same host arrays. This module holds no arithmetic
of the method itself (no top-k sum, no residual add, no normalisation); it only
draws random tensors of the shapes and distributions of the decode workloads
and rounds them to bf16 with torch's converter.

Workloads (shapes from the pages, distributions chosen for this library):
  * tokens per decode step 1/4/12/28 (1, 3 or 7 requests times 4 MTP tokens)
    plus 64, and a 512-token batch at the CUDA-graph capture ceiling
    ("Port the validated GLM-5.2 H200 production path to latest vLLM",
    Prepared experiment branches);
  * an 8192-token prefill chunk (same page, Resume protocol);
  * hidden 6144 (same page, the GEMM2 n of the MoE) and 2048, top-8 routing
    ("vLLM pull request #62174", Validation: tokens 1, 4, 64 and hidden
    2048/6144 in its fused all-reduce RMSNorm test).

Generator: numpy PCG64 with seed = 20261202 + 1000*seed_index + T (each named
workload has a seed index); SeedSequence(seed)
spawns one child stream per tensor, in the order expert_out, perm, logits,
shared, residual, gamma, mask, spikes. Normals are drawn in float32, scaled as
mu + sigma*z in float32, then rounded to bf16 (round-to-nearest-even).
"""
import math

import numpy as np
import torch

BASE_SEED = 20261202
STREAMS = ("expert_out", "perm", "logits", "shared", "residual", "gamma", "mask", "spikes")

# Workload recipes, by name. Ts lists the token counts each is run at; seed_index
# enters the seed (seed = 20261202 + 1000 * seed_index + T).
CONFIGS = {
    "tiny": dict(seed_index=0, Ts=(4,), H=2048, K=8, scale=1.0, weights="softmax_k",
                 mask_frac=0.0, spike_frac=0.0, name="tiny: T=4 H=2048 K=8"),
    "decode": dict(seed_index=1, Ts=(1, 4, 12, 28, 64), H=6144, K=8, scale=2.5,
                   weights="softmax_k", mask_frac=0.0, spike_frac=0.0,
                   name="decode latency sweep: H=6144 K=8"),
    "decode_masked": dict(seed_index=2, Ts=(1, 4, 64), H=2048, K=8, scale=2.5, weights="softmax_k",
                          mask_frac=0.05, spike_frac=0.0,
                          name="small-hidden decode, 5% masked slots: H=2048 K=8"),
    "batch512": dict(seed_index=3, Ts=(512,), H=6144, K=8, scale=2.5, weights="top8_of_256",
                     mask_frac=0.0, spike_frac=0.0,
                     name="batched decode at graph ceiling: T=512 H=6144 K=8"),
    "prefill": dict(seed_index=4, Ts=(8192,), H=6144, K=8, scale=2.5, weights="top8_of_256",
                    mask_frac=0.0, spike_frac=0.01,
                    name="prefill chunk: T=8192 H=6144 K=8, 1% residual rows x100"),
}
EPS = 1e-6
_CHUNK = 1 << 22  # values per float32 chunk when drawing large tensors


def seed_for(cfg, T):
    """Seed of a named workload at token count T."""
    return BASE_SEED + 1000 * CONFIGS[cfg]["seed_index"] + T


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest-even, torch's converter); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b):
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng, shape, mu, sigma):
    """Draw N(mu, sigma^2) in float32 and round to bf16 bits, in row chunks."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    if out.size == 0:
        return out
    flat = out.reshape(-1)
    mu = np.float32(mu)
    sigma = np.float32(sigma)
    for lo in range(0, flat.size, _CHUNK):
        hi = min(flat.size, lo + _CHUNK)
        z = rng.standard_normal(hi - lo, dtype=np.float32)
        flat[lo:hi] = f32_to_bf16_bits(mu + sigma * z)
    return out


def _softmax64(logits):
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def expert_sorted_perm(experts):
    """perm_idx [T, K] of the expert-sorted row layout, from the expert each
    (token, slot) picked: a pair's row is its rank when the pairs are sorted
    by expert, ties (one expert, several tokens) in token order."""
    experts = np.asarray(experts)
    n = experts.size
    by_expert = np.argsort(experts.reshape(-1), kind="stable")
    flat = np.empty(n, dtype=np.int32)
    flat[by_expert] = np.arange(n, dtype=np.int32)
    return flat.reshape(experts.shape)


def generate(T, H, K, *, scale=2.5, eps=EPS, weights="softmax_k", mask_frac=0.0,
             spike_frac=0.0, seed=BASE_SEED, extra_rows=0, layout="random"):
    """Draw one input set.

    weights: "softmax_k"   - softmax over the K slots of N(0,1) logits;
             "top8_of_256" - softmax over the K largest of 256 N(0,1) logits
                             (ties go to the lower expert index).
    layout: "random"        - the rows of expert_out in a uniformly random order;
            "expert_sorted" - grouped by the expert each (token, slot) picked,
                              tokens in order within an expert: the layout of a
                              grouped GEMM2 output (needs "top8_of_256"; every
                              other array is the same as with "random").
    mask_frac: fraction of (token, slot) pairs masked, rounded up; masked pairs get
               perm_idx = -1 and weight 0, and each token's remaining weights are
               renormalised to sum to 1 (an all-masked token keeps zero weights).
    spike_frac: fraction of residual rows (rounded) multiplied by 100 before rounding.
    extra_rows: rows appended to expert_out that no index refers to.
    """
    T, H, K = int(T), int(H), int(K)
    ss = np.random.SeedSequence(seed)
    rng = dict(zip(STREAMS, [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(len(STREAMS))]))
    R = T * K + int(extra_rows)

    expert_out = _normal_bf16(rng["expert_out"], (R, H), 0.0, 1.0)
    perm = rng["perm"].permutation(T * K).astype(np.int32).reshape(T, K)

    order = None
    if weights == "softmax_k":
        logits = rng["logits"].standard_normal((T, K), dtype=np.float32)
        w64 = _softmax64(logits)
    elif weights == "top8_of_256":
        n_exp = 256
        if K > n_exp:
            raise ValueError("K exceeds the 256 experts")
        logits = rng["logits"].standard_normal((T, n_exp), dtype=np.float32)
        order = np.argsort(-logits, axis=1, kind="stable")[:, :K]
        w64 = _softmax64(np.take_along_axis(logits, order, axis=1))
    else:
        raise ValueError(f"unknown weights recipe {weights!r}")
    if layout == "expert_sorted":
        if weights != "top8_of_256":
            raise ValueError("the expert_sorted layout needs the experts of top8_of_256")
        perm = expert_sorted_perm(order)
    elif layout != "random":
        raise ValueError(f"unknown layout {layout!r}")

    if mask_frac > 0 and T * K > 0:
        m = int(math.ceil(mask_frac * T * K))
        flat = rng["mask"].choice(T * K, size=m, replace=False)
        mask = np.zeros(T * K, dtype=bool)
        mask[flat] = True
        mask = mask.reshape(T, K)
        perm[mask] = -1
        w64[mask] = 0.0
        tot = w64.sum(axis=1, keepdims=True)
        w64 = np.where(tot > 0, w64 / np.where(tot > 0, tot, 1.0), 0.0)
    topk_w = w64.astype(np.float32)

    shared = _normal_bf16(rng["shared"], (T, H), 0.0, 0.5)
    if spike_frac > 0 and T > 0:
        n_spike = int(round(spike_frac * T))
        spike_rows = np.sort(rng["spikes"].choice(T, size=n_spike, replace=False))
        resid = np.empty((T, H), dtype=np.uint16)
        rr = rng["residual"]
        spike = np.zeros(T, dtype=bool)
        spike[spike_rows] = True
        rows_per = max(1, _CHUNK // max(H, 1))
        for lo in range(0, T, rows_per):
            hi = min(T, lo + rows_per)
            z = rr.standard_normal((hi - lo, H), dtype=np.float32)
            x = np.float32(4.0) * z
            x[spike[lo:hi]] *= np.float32(100.0)
            resid[lo:hi] = f32_to_bf16_bits(x)
    else:
        spike_rows = np.zeros(0, dtype=np.int64)
        resid = _normal_bf16(rng["residual"], (T, H), 0.0, 4.0)
    gamma = _normal_bf16(rng["gamma"], (H,), 1.0, 0.1)

    return dict(expert_out=expert_out, perm_idx=perm, topk_w=topk_w, shared_out=shared,
                residual=resid, gamma=gamma, eps=float(np.float32(eps)),
                scale=float(np.float32(scale)), T=T, H=H, K=K, R=R, spike_rows=spike_rows,
                experts=None if order is None else order.astype(np.int32))


def dense_inputs(T, H, *, eps=EPS, seed=BASE_SEED, spike_frac=0.0):
    """Inputs of the dense residual add + RMSNorm: x (a row-parallel layer
    output, N(0, 0.5^2), drawn like shared_out) and residual (N(0, 4^2), with
    the optional x100 rows) from the same streams as generate()."""
    d = generate(T, H, 1, eps=eps, seed=seed, spike_frac=spike_frac)
    return dict(x=d["shared_out"], residual=d["residual"], gamma=d["gamma"], eps=d["eps"], T=T,
                H=H, spike_rows=d["spike_rows"])


def fp8_algorithmic_bytes(perm_idx, H, K, bf16_normed=False):
    """The fused op writing its normalised output as FP8: the reads of
    algorithmic_bytes, residual_out (2H), the E4M3 codes (H) and the scale (4)
    per token, plus the bf16 normed output (2H) when it is also written."""
    T = perm_idx.shape[0]
    valid = int((np.asarray(perm_idx) >= 0).sum())
    per_token_out = 2 * H + H + 4 + (2 * H if bf16_normed else 0)
    return 2 * H * valid + 2 * (2 * H) * T + 8 * K * T + 2 * H + per_token_out * T


def dense_algorithmic_bytes(T, H):
    """x, residual and both outputs (2H bytes each per token), plus gamma once."""
    return 8 * H * T + 2 * H


def dense_fp8_algorithmic_bytes(T, H, bf16_normed=False):
    """The dense tail writing its normalised output as FP8: x, residual and
    residual_out (2H bytes each per token), the E4M3 codes (H) and the scale
    (4) per token, the bf16 normed output (2H) when it is also written, plus
    gamma once."""
    return (6 * H + H + 4 + (2 * H if bf16_normed else 0)) * T + 2 * H


def config_inputs(cfg, T=None):
    """Inputs of a named workload config at token count T (default: its first T)."""
    c = CONFIGS[cfg]
    if T is None:
        T = c["Ts"][0]
    return generate(T, c["H"], c["K"], scale=c["scale"], weights=c["weights"],
                    mask_frac=c["mask_frac"], spike_frac=c["spike_frac"], seed=seed_for(cfg, T))


def config_algorithmic_bytes(cfg, T):
    """algorithmic_bytes of a named workload with no masked slots, without
    drawing its inputs (every slot is valid: T * K gathered rows)."""
    c = CONFIGS[cfg]
    if c["mask_frac"] != 0.0:
        raise ValueError(f"{cfg} masks slots: count them with algorithmic_bytes")
    H, K = c["H"], c["K"]
    return 2 * H * T * K + 4 * (2 * H) * T + 8 * K * T + 2 * H


def config_fp8_algorithmic_bytes(cfg, T, bf16_normed=False):
    """fp8_algorithmic_bytes of a named workload with no masked slots, without
    drawing its inputs."""
    c = CONFIGS[cfg]
    if c["mask_frac"] != 0.0:
        raise ValueError(f"{cfg} masks slots: count them with fp8_algorithmic_bytes")
    H, K = c["H"], c["K"]
    per_token_out = 2 * H + H + 4 + (2 * H if bf16_normed else 0)
    return 2 * H * T * K + 2 * (2 * H) * T + 8 * K * T + 2 * H + per_token_out * T


def algorithmic_bytes(perm_idx, H, K):
    """Bytes the op must move: valid gathered rows, shared, residual, both
    outputs (2H bytes each per token), the K index and K weight entries per
    token, and gamma once."""
    T = perm_idx.shape[0]
    valid = int((np.asarray(perm_idx) >= 0).sum())
    return 2 * H * valid + 4 * (2 * H) * T + 8 * K * T + 2 * H
