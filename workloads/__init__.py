"""Seeded synthetic inputs shared by the oracle side and the HIP side of the tests and bench.

This module only draws numbers: it holds none of the quantization or GEMM
arithmetic, and neither the oracle nor the HIP library is imported here.

Recipe (the pages name no dataset; these stand in for the activations,
weights and gradients of one FP8 Linear layer and of one MoE expert layer):

* generator: ``numpy.random.default_rng(seed)`` (PCG64);
* values: float32 draws ``sigma * standard_normal`` in row-major order;
* outliers (the pages motivate tile/block scaling by activation outliers):
  ``round(frac * numel)`` distinct positions from ``rng.choice`` are multiplied
  by ``factor`` (sign kept);
* BF16 tensors: the float32 draw rounded to nearest-even BF16 (via torch's
  CPU cast), handed around as uint16 bit patterns;
* "N(0, s)" means standard deviation s.
"""

import numpy as np

GROUP = 128


def _torch():
    import torch
    return torch


def normal_f32(rng, shape, sigma):
    """sigma * N(0,1) as float32, drawn in float32 in row-major order."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def add_outliers(rng, x, frac, factor):
    """Multiply round(frac*numel) distinct entries of x (in place) by factor."""
    flat = x.reshape(-1)
    n = int(round(frac * flat.size))
    if n:
        idx = rng.choice(flat.size, size=n, replace=False)
        flat[idx] *= np.float32(factor)
    return x


def to_bf16_bits(x_f32):
    """Nearest-even BF16 bit patterns (uint16) of a float32 array."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_as_f32(bits):
    """Float32 values of BF16 bit patterns (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Named workloads
# ----------------------------------------------------------------------------

def tiny_fprop(seed=1):
    """A 128x256 fp32 N(0,1) with 0.5% entries x100; B 256x128 fp32 N(0,0.02).

    B is the logical [K][N] weight; the GEMM consumes it K-contiguous, as
    Bt = B.T of shape [N][K]. Returns dict(a=A, bt=Bt), both float32.
    """
    rng = np.random.default_rng(seed)
    a = add_outliers(rng, normal_f32(rng, (128, 256), 1.0), 0.005, 100.0)
    b = normal_f32(rng, (256, 128), 0.02)
    return {"a": a, "bt": np.ascontiguousarray(b.T)}


def linear_layer(seed=2, tokens=8192, d_in=7168, d_out=18432):
    """Activation X [tokens][d_in] bf16 N(0,1) + 0.1% x50 outliers and the weight
    stored as Wt [d_out][d_in] bf16 N(0,0.02). Returns bf16 bit arrays."""
    rng = np.random.default_rng(seed)
    x = add_outliers(rng, normal_f32(rng, (tokens, d_in), 1.0), 0.001, 50.0)
    xb = to_bf16_bits(x)
    del x
    wt = normal_f32(rng, (d_out, d_in), 0.02)
    wb = to_bf16_bits(wt)
    return {"x": xb, "wt": wb}


def output_grad(seed=4, tokens=8192, d_out=18432):
    """dY [tokens][d_out] bf16 N(0, 1e-3)."""
    rng = np.random.default_rng(seed)
    return {"dy": to_bf16_bits(normal_f32(rng, (tokens, d_out), 1e-3))}


def moe_group_sizes(seed=5, groups=64, tokens=65536, zipf_s=1.1):
    """Per-expert token counts ~ Multinomial(tokens, p_i ~ i^-s), i = 1..groups
    (unshuffled: group 0 is the largest). Returns (rng, counts)."""
    rng = np.random.default_rng(seed)
    p = np.arange(1, groups + 1, dtype=np.float64) ** (-zipf_s)
    p /= p.sum()
    counts = rng.multinomial(tokens, p)
    return rng, counts


def moe_layer(seed=5, groups=64, tokens=65536, d_in=7168, d_out=2048, zipf_s=1.1):
    """Grouped MoE expert layer.

    Per-group token counts as in ``moe_group_sizes``; each group's activation
    slab (counts_e x d_in, N(0,1) with 0.1% x50 outliers) is padded with zero
    rows to a multiple of 128 and the slabs are concatenated; each expert's
    weight is stored [d_out][d_in] ~ N(0,0.02) and the experts are stacked.
    Returns dict(x=bf16 bits [M_pad][d_in], wt=bf16 bits [G*d_out][d_in],
    counts, padded (per-group padded rows), group_of_mtile (int32)).
    """
    rng, counts = moe_group_sizes(seed, groups, tokens, zipf_s)
    padded = [(-(-int(c) // GROUP)) * GROUP for c in counts]
    m_pad = int(sum(padded))
    x = np.zeros((m_pad, d_in), dtype=np.uint16)
    row = 0
    for c, pc in zip(counts, padded):
        if c:
            slab = add_outliers(rng, normal_f32(rng, (int(c), d_in), 1.0), 0.001, 50.0)
            x[row:row + int(c)] = to_bf16_bits(slab)
        row += pc
    wt = np.empty((groups * d_out, d_in), dtype=np.uint16)
    for e in range(groups):
        wt[e * d_out:(e + 1) * d_out] = to_bf16_bits(normal_f32(rng, (d_out, d_in), 0.02))
    gmap = np.concatenate([np.full(pc // GROUP, e, dtype=np.int32)
                           for e, pc in enumerate(padded)]) if m_pad else np.zeros(0, np.int32)
    return {"x": x, "wt": wt, "counts": np.asarray(counts), "padded": np.asarray(padded),
            "group_of_mtile": gmap}


def random_fp8_operands(seed, m, n, k, kind="fprop", scale_lo=2.0 ** -12, scale_hi=2.0 ** -2, pow2=False):
    """Random non-NaN E4M3 codes and positive float32 scales for direct GEMM tests.

    Codes are uniform over the 254 non-NaN bytes; scales are log-uniform in
    [scale_lo, scale_hi] (pow2=True: their exponents rounded to integers, so
    every scale is a power of two). Scale layouts: sa [K/128][M]; sb
    [N/128][K/128] (fprop/dgrad) or [K/128][N] (wgrad).
    """
    rng = np.random.default_rng(seed)
    valid = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    qa = valid[rng.integers(0, valid.size, size=(m, k))]
    qb = valid[rng.integers(0, valid.size, size=(n, k))]
    g = -(-k // GROUP)
    lo, hi = np.log2(scale_lo), np.log2(scale_hi)
    expo = (lambda e: np.rint(e)) if pow2 else (lambda e: e)
    sa = np.exp2(expo(rng.uniform(lo, hi, size=(g, m)))).astype(np.float32)
    if kind == "wgrad":
        sb = np.exp2(expo(rng.uniform(lo, hi, size=(g, n)))).astype(np.float32)
    else:
        sb = np.exp2(expo(rng.uniform(lo, hi, size=(-(-n // GROUP), g)))).astype(np.float32)
    return {"qa": qa, "sa": sa, "qb": qb, "sb": sb}


# ----------------------------------------------------------------------------
# Device-side draws for tensors too large to stage through the host (beyond
# 2^31 elements); the tests copy the sampled parts back for the oracle.
# ----------------------------------------------------------------------------

def device_normal_bf16(seed, shape, sigma=1.0):
    """sigma * N(0,1) drawn on the GPU by torch's seeded CUDA generator, rounded to BF16."""
    torch = _torch()
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)
    if sigma != 1.0:
        x.mul_(sigma)
    return x


def device_fp8_codes(seed, shape):
    """Uniform random bytes drawn on the GPU; the two NaN codes (0x7F, 0xFF) are
    moved to their neighbours 0x7E / 0xFE, so every byte is a finite E4M3 code."""
    torch = _torch()
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randint(0, 256, shape, generator=g, device="cuda", dtype=torch.uint8)
    q.sub_(((q & 0x7F) == 0x7F).to(torch.uint8))    # elementwise (masked indexing fails past 2^31 elements)
    return q
