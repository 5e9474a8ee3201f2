"""Seeded synthetic inputs for the block-scaled FP4 expert MLP.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantisation, dequantisation or GEMM). Both the CPU
oracle and the GPU library are fed from here.

Shapes follow the pages' expert format ("2026-05-08 DeepSeek V4 Pro NVFP4
Quantization", section "FP4 (E2M1) expert weight format confirmed": w1/w3
packed [3072, 3584] with E8M0 [3072, 224], w2 packed [7168, 1536] with E8M0
[7168, 96]) and the 48 local experts per rank of "Current Bug: vLLM produces
empty/garbage output", section "Config values". The pages use real checkpoint
weights, which are not available: every tensor here is synthetic.

Recipes (numpy ``default_rng``):
* packed E2M1 codes: independent uniform bytes (every nibble uniform over 16);
* E8M0 scales: integers uniform in an inclusive exponent range;
* activations: N(0, 1) in fp32 rounded to bf16 by torch's cast;
* routing: k distinct experts per token, fp32 softmax of N(0, 1) logits as
  gate weights (the router is outside the method: ids and weights are inputs);
* skewed routing: expert popularity p_i ~ rank**-s over a random permutation,
  the lowest-ranked experts get p = 0, k distinct experts drawn without
  replacement in proportion to p (Gumbel top-k).
"""

from __future__ import annotations

import numpy as np

HIDDEN = 7168
INTER = 3072
N_LOCAL_EXPERTS = 48
TOP_K = 8


def _bf16_bits(f32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(rng, shape):
    """bf16 bit patterns of N(0, 1) samples."""
    return _bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def packed_codes(rng, shape):
    """Uniform random bytes of the given packed shape (two E2M1 codes each)."""
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def e8m0_scales(rng, shape, lo, hi):
    """E8M0 scale bytes uniform over the exponent bytes lo..hi inclusive."""
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def mxfp4_weight(rng, rows, cols, lo=120, hi=130, lead=()):
    """One MXFP4 matrix of logical shape [rows, cols]: (codes, scales)."""
    return (packed_codes(rng, lead + (rows, cols // 2)),
            e8m0_scales(rng, lead + (rows, cols // 32), lo, hi))


def expert_weights(seed, hidden=HIDDEN, inter=INTER, n_experts=None, lo=120, hi=130):
    """w1, w1s, w3, w3s, w2, w2s for one expert (n_experts=None) or a stack."""
    rng = np.random.default_rng(seed)
    lead = () if n_experts is None else (n_experts,)
    w1, w1s = mxfp4_weight(rng, inter, hidden, lo, hi, lead)
    w3, w3s = mxfp4_weight(rng, inter, hidden, lo, hi, lead)
    w2, w2s = mxfp4_weight(rng, hidden, inter, lo, hi, lead)
    return dict(w1=w1, w1s=w1s, w3=w3, w3s=w3s, w2=w2, w2s=w2s)


def activations(seed, tokens, hidden=HIDDEN):
    return bf16_normal(np.random.default_rng(seed), (tokens, hidden))


def uniform_routing(seed, tokens, n_experts=N_LOCAL_EXPERTS, k=TOP_K):
    """k distinct experts per token chosen uniformly; softmax gate weights."""
    rng = np.random.default_rng(seed)
    keys = rng.random((tokens, n_experts))
    ids = np.argsort(keys, axis=1)[:, :k].astype(np.int32)
    logits = rng.standard_normal((tokens, k)).astype(np.float32)
    return ids, _softmax_f32(logits)


def zipf_routing(seed, tokens, n_experts=N_LOCAL_EXPERTS, k=TOP_K, s=1.2, n_empty=4):
    """Skewed routing: popularity ~ rank**-s, the last n_empty ranks never chosen."""
    rng = np.random.default_rng(seed)
    ranks = np.arange(1, n_experts + 1, dtype=np.float64)
    p_rank = ranks ** -s
    p_rank[n_experts - n_empty:] = 0.0
    perm = rng.permutation(n_experts)
    p = np.zeros(n_experts)
    p[perm] = p_rank / p_rank.sum()
    with np.errstate(divide="ignore"):
        logp = np.log(p)
    gumbel = rng.gumbel(size=(tokens, n_experts))
    ids = np.argsort(-(logp[None, :] + gumbel), axis=1)[:, :k].astype(np.int32)
    logits = rng.standard_normal((tokens, k)).astype(np.float32)
    return ids, _softmax_f32(logits)


def _softmax_f32(logits):
    z = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(z, dtype=np.float32)
    return (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def e4m3_finite_codes(rng, shape):
    """Bytes uniform over the 254 finite float8_e4m3fn codes (0x7F, 0xFF excluded)."""
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    return finite[rng.integers(0, finite.size, size=shape)]


# ---------------------------------------------------------------------------
# The named workloads
# ---------------------------------------------------------------------------

def tiny_mlp(seed=0):
    """Single expert, hidden 256, intermediate 128, 16 tokens, one seed."""
    rng = np.random.default_rng(seed)
    w1, w1s = mxfp4_weight(rng, 128, 256)
    w3, w3s = mxfp4_weight(rng, 128, 256)
    w2, w2s = mxfp4_weight(rng, 256, 128)
    x = bf16_normal(rng, (16, 256))
    return dict(x=x, w1=w1, w1s=w1s, w3=w3, w3s=w3s, w2=w2, w2s=w2s, hidden=256, inter=128)


def dequant_inputs(seed=0, lo=118, hi=134):
    """Real-shape dequant inputs: w1-like, w2-like MXFP4 and an FP8 128x128-block matrix."""
    rng = np.random.default_rng(seed)
    w1, w1s = mxfp4_weight(rng, INTER, HIDDEN, lo, hi)
    w2, w2s = mxfp4_weight(rng, HIDDEN, INTER, lo, hi)
    q = e4m3_finite_codes(rng, (HIDDEN, 1536))
    qs = e8m0_scales(rng, (HIDDEN // 128, 1536 // 128), lo, hi)
    return dict(w1=w1, w1s=w1s, w2=w2, w2s=w2s, fp8=q, fp8s=qs)


def shared_expert(tokens, seed=0, hidden=HIDDEN, inter=INTER):
    """Shared expert: one MXFP4 expert (weights seed, activations seed + 1)."""
    d = expert_weights(seed, hidden, inter)
    d["x"] = activations(seed + 1, tokens, hidden)
    return d


def grouped(tokens=4096, n_experts=N_LOCAL_EXPERTS, k=TOP_K, seed=0,
            hidden=HIDDEN, inter=INTER):
    """Routed experts, uniform top-k (weights seed, x seed + 1, routing seed + 2)."""
    d = expert_weights(seed, hidden, inter, n_experts)
    d["x"] = activations(seed + 1, tokens, hidden)
    d["ids"], d["w"] = uniform_routing(seed + 2, tokens, n_experts, k)
    return d


def skewed(tokens=16384, n_experts=N_LOCAL_EXPERTS, k=TOP_K, seed=0,
           hidden=HIDDEN, inter=INTER):
    """Routed experts with Zipf(1.2) popularity and 4 experts never chosen."""
    d = expert_weights(seed, hidden, inter, n_experts)
    d["x"] = activations(seed + 1, tokens, hidden)
    d["ids"], d["w"] = zipf_routing(seed + 2, tokens, n_experts, k)
    return d


def fp8_linear(tokens, n=HIDDEN, k=1536, seed=0, lo=118, hi=134):
    """FP8 block-scaled linear: E4M3 weights [n, k] uniform over the finite codes,
    E8M0 128 x 128 block scales uniform in [lo, hi] (weights seed), bf16
    activations N(0, 1) [tokens, k] (seed + 1). The default shape is the pages'
    FP8 matrix [7168, 1536]."""
    rng = np.random.default_rng(seed)
    w = e4m3_finite_codes(rng, (n, k))
    ws = e8m0_scales(rng, (n // 128, k // 128), lo, hi)
    return dict(w=w, ws=ws, x=activations(seed + 1, tokens, k))


def fp8_expert(tokens, hidden=HIDDEN, inter=INTER, seed=0, lo=112, hi=120):
    """FP8 shared expert: E4M3 w1, w3 [inter, hidden] and w2 [hidden, inter] uniform
    over the finite codes with 128 x 128 E8M0 block scales uniform in [lo, hi]
    (weights seed; the lower exponents keep the gate values near the SiLU's
    active range for N(0, 1) inputs), bf16 activations N(0, 1) (seed + 1)."""
    rng = np.random.default_rng(seed)
    d = {}
    for n, (r, c) in (("w1", (inter, hidden)), ("w3", (inter, hidden)), ("w2", (hidden, inter))):
        d[n] = e4m3_finite_codes(rng, (r, c))
        d[n + "s"] = e8m0_scales(rng, (r // 128, c // 128), lo, hi)
    d["x"] = activations(seed + 1, tokens, hidden)
    return d


def nvfp4_linear(tokens, n=HIDDEN, k=INTER, seed=0):
    """NVFP4-weight linear: E2M1 code bytes uniform (all 16 nibbles), E4M3 block
    scales uniform over the codes with exponent field 4..10 (2^-3 .. 2^3 times
    the mantissa), fp32 weight global 2^-6 (weights seed); bf16 activations
    N(0, 1) [tokens, k] (seed + 1) with the fixed activation global 2^-9 (a
    block maximum up to 6 * 448 * 2^-9 = 5.25 needs no saturation). The default
    shape is the down projection [7168, 3072]."""
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 256, (n, k // 2)).astype(np.uint8)
    ws = rng.integers(0x20, 0x58, (n, k // 16)).astype(np.uint8)
    return dict(w=w, ws=ws, wg=np.float32(2.0 ** -6), x=activations(seed + 1, tokens, k), xg=np.float32(2.0 ** -9))


def nvfp4_linear_wide(tokens, n, k, seed=0):
    """``nvfp4_linear`` with the E4M3 weight scales uniform over every finite
    byte (0x00 .. 0x7E: zero, the subnormals up to 448) and each 16-block of
    activations N(0, 1) times 2^e, e uniform in -20 .. 4, so that the
    activations' own block scales reach zero, the subnormals and saturation."""
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 256, (n, k // 2)).astype(np.uint8)
    ws = rng.integers(0x00, 0x7F, (n, k // 16)).astype(np.uint8)
    e = rng.integers(-20, 5, (tokens, k // 16)).repeat(16, axis=1)
    x = _bf16_bits((rng.standard_normal((tokens, k)) * np.exp2(e)).astype(np.float32))
    return dict(w=w, ws=ws, wg=np.float32(2.0 ** -6), x=x, xg=np.float32(2.0 ** -9))


def nvfp4_expert(tokens, hidden=HIDDEN, inter=INTER, seed=0):
    """One expert with NVFP4 weights: codes and E4M3 scales as ``nvfp4_linear``,
    weight globals 2^-6 (w1), 2^-5 (w3, a different one: the dual gate/up
    globals) and 2^-6 (w2) (weights seed); bf16 activations N(0, 1) (seed + 1)
    with activation global 2^-9 and intermediate global 1."""
    rng = np.random.default_rng(seed)
    d = {}
    for n, (r, c) in (("w1", (inter, hidden)), ("w3", (inter, hidden)), ("w2", (hidden, inter))):
        d[n] = rng.integers(0, 256, (r, c // 2)).astype(np.uint8)
        d[n + "s"] = rng.integers(0x20, 0x58, (r, c // 16)).astype(np.uint8)
    d.update(w1g=np.float32(2.0 ** -6), w3g=np.float32(2.0 ** -5), w2g=np.float32(2.0 ** -6),
             xg=np.float32(2.0 ** -9), hg=np.float32(1.0), x=activations(seed + 1, tokens, hidden))
    return d


def grouped_nvfp4(tokens=4096, n_experts=N_LOCAL_EXPERTS, k=TOP_K, seed=0, hidden=HIDDEN, inter=INTER):
    """Routed experts with NVFP4 weights: per expert, codes and E4M3 scales as
    ``nvfp4_linear`` and fp32 globals 2^-6 * (1 + (e mod 4) / 4) for w1,
    2^-5 * (1 + (e mod 3) / 3) for w3 and 2^-6 for w2 (weights seed);
    activations N(0, 1) (seed + 1) with globals 2^-9 (x) and 1 (h); uniform
    top-k routing (seed + 2)."""
    rng = np.random.default_rng(seed)
    d = {}
    for n, (r, c) in (("w1", (inter, hidden)), ("w3", (inter, hidden)), ("w2", (hidden, inter))):
        d[n] = rng.integers(0, 256, (n_experts, r, c // 2), dtype=np.uint8)
        d[n + "s"] = rng.integers(0x20, 0x58, (n_experts, r, c // 16), dtype=np.uint8)
    e = np.arange(n_experts)
    d["w1g"] = (2.0 ** -6 * (1 + (e % 4) / 4)).astype(np.float32)
    d["w3g"] = (2.0 ** -5 * (1 + (e % 3) / 3)).astype(np.float32)
    d["w2g"] = np.full(n_experts, 2.0 ** -6, np.float32)
    d["xg"], d["hg"] = np.float32(2.0 ** -9), np.float32(1.0)
    d["x"] = activations(seed + 1, tokens, hidden)
    d["ids"], d["w"] = uniform_routing(seed + 2, tokens, n_experts, k)
    return d

