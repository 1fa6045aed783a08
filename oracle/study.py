"""Quantization-error study of the scaling rules (TEST INFRASTRUCTURE ONLY --
never imported by the product path).

Compares, on the outlier-bearing synthetic tensors, the relative Frobenius
error ||deq(q) - x|| / ||x|| of:
  * per-tensor max-abs scaling (one scale for the whole tensor): the common
    practice whose outlier sensitivity motivates fine-grained scaling
    ("Deepseek - Not For everyone", paragraph 3);
  * 1x128 tiles and 128x128 blocks (dssusan.co.kr FP8 excerpt, paragraphs 2
    and 4), with max-abs and power-of-2 scales (paragraph 1);
  * delayed (history) max-abs scaling, where the scale comes from the max-abs
    of earlier iterations rather than the current tensor (the tensor-wise
    scheme the pages contrast with their online one, dssusan.co.kr paragraph
    2), on a sequence whose magnitude drifts between iterations.
Everything is built from the pinned oracle quantizers plus the plain rule of
each alternative; run ``python -m oracle.study`` for the table.
"""

import numpy as np

from . import e4m3, quant

F448 = np.float32(448.0)


def rel_error(deq, x):
    x = np.asarray(x, np.float64)
    return float(np.linalg.norm(np.asarray(deq, np.float64) - x) / np.linalg.norm(x))


def underflow_fraction(q, x):
    """Share of nonzero inputs whose code is +-0."""
    nz = np.asarray(x) != 0
    return float(np.mean((np.asarray(q) & 0x7F)[nz] == 0))


def quant_with_scale(x, s, inv):
    """Quantize with a given scale pair (per-tensor / delayed rules): clamp to
    +-448 after the multiply, then E4M3 round-to-nearest-even."""
    y = (np.asarray(x, np.float32) * np.float32(inv)).astype(np.float32)
    return e4m3.encode(np.clip(y, -F448, F448)), np.float32(s)


def per_tensor(x, mode=quant.MODE_MAXABS):
    s, inv = quant.scales_from_amax(np.max(np.abs(x)), mode)
    q, s = quant_with_scale(x, s, inv)
    return q, s, e4m3.decode(q) * np.float64(s)


def fine_1x128(x, mode):
    q, s = quant.quant_1x128(x, mode)
    return q, s, quant.dequant_1x128(q, s)


def fine_128x128(x, mode):
    q, s = quant.quant_128x128(x, mode)
    return q, s, quant.dequant_128x128(q, s)


def delayed_sequence(xs, history=16, mode=quant.MODE_MAXABS):
    """Delayed per-tensor scaling over iterations: the scale of iteration t is
    derived from max(amax of iterations t-history .. t-1) (the first iteration
    uses its own max-abs).  Returns the per-iteration relative errors and the
    share of elements clipped at +-448."""
    amaxes, errs, clipped = [], [], []
    for t, x in enumerate(xs):
        a_now = np.float32(np.max(np.abs(x)))
        a = np.float32(max(amaxes[-history:])) if amaxes else a_now
        s, inv = quant.scales_from_amax(a, mode)
        q, s = quant_with_scale(x, s, inv)
        errs.append(rel_error(e4m3.decode(q) * np.float64(s), x))
        clipped.append(float(np.mean(np.abs(np.asarray(x, np.float32) * np.float32(inv)) > F448)))
        amaxes.append(a_now)
    return errs, clipped


def table(seed=0, rows=1024):
    """Error table on slices of the synthetic workloads (rows of each tensor)."""
    from workloads import bf16_bits_as_f32, linear_layer, output_grad, tiny_fprop
    lin = linear_layer()
    tensors = {
        "activation X (N(0,1), 0.1% x50 outliers)": bf16_bits_as_f32(lin["x"][:rows]),
        "weight W (N(0,0.02))": bf16_bits_as_f32(lin["wt"][:rows]),
        "output grad dY (N(0,1e-3))": bf16_bits_as_f32(output_grad()["dy"][:rows, :7168]),
        "tiny A (N(0,1), 0.5% x100 outliers)": tiny_fprop()["a"],
    }
    out = []
    for name, x in tensors.items():
        row = {"tensor": name}
        for mode in (quant.MODE_MAXABS, quant.MODE_POW2):
            q, _, d = per_tensor(x, mode)
            row[f"per-tensor {mode}"] = (rel_error(d, x), underflow_fraction(q, x))
            q, _, d = fine_1x128(x, mode)
            row[f"1x128 {mode}"] = (rel_error(d, x), underflow_fraction(q, x))
            q, _, d = fine_128x128(x, mode)
            row[f"128x128 {mode}"] = (rel_error(d, x), underflow_fraction(q, x))
        out.append(row)
    # delayed scaling on an activation sequence: each iteration is a fresh
    # shuffle of the same rows, and iteration 5 carries a spike (0.01% of the
    # entries set to +-4x the tensor's usual max-abs) that the history has not seen
    rng = np.random.default_rng(seed)
    base = bf16_bits_as_f32(lin["x"][:256])
    xs = []
    for t in range(8):
        x = base[rng.permutation(base.shape[0])].copy()
        if t == 5:
            flat = x.reshape(-1)
            idx = rng.choice(flat.size, flat.size // 10000, replace=False)
            flat[idx] = np.sign(flat[idx]) * np.float32(4.0) * np.max(np.abs(base))
        xs.append(x)
    errs, clipped = delayed_sequence(xs, history=4)
    online = [rel_error(fine_1x128(x, quant.MODE_MAXABS)[2], x) for x in xs]
    return out, {"delayed per-tensor": errs, "delayed clipped share": clipped, "online 1x128": online}


def _main():
    rows, delayed = table()
    cols = [c for c in rows[0] if c != "tensor"]
    print("| tensor | " + " | ".join(cols) + " |")
    print("|---" * (len(cols) + 1) + "|")
    for r in rows:
        print(f"| {r['tensor']} | " + " | ".join(f"{r[c][0]:.4f} ({100 * r[c][1]:.2f}% zero)" for c in cols) + " |")
    print()
    for k, v in delayed.items():
        print(k, " ".join(f"{e:.4f}" for e in v))


if __name__ == "__main__":
    _main()
