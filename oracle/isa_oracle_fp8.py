"""FP8 (e4m3) variant of the ISA full route, on the CPU (test infrastructure).

TEST INFRASTRUCTURE ONLY; shares no code with the HIP kernels.

The pages mention 8-bit quantisation as a way to speed attention up ("8-bit
quantisation" among the optimisations listed on the first page); the FP8
variant of the full route computes the same exact attention as R8 of
isa_oracle.py with its operands rounded to the OCP e4m3 format under
power-of-two block scales (the MX convention of a shared 2^e per block of 32
elements):
  Q   per (query row, 32 consecutive d)
  K   per (key row, 32 consecutive d)
  V   per (d, 32 consecutive keys of the full route's key list, counted from
      its start: source rows, then the tokens of the kept context blocks)
  P   the probabilities exp(l - m) with m the row's maximum logit rounded up
      to a whole power of two in the exp2 domain, unscaled.
The block exponent is the smallest e with max|x| / 2^e <= 448 (e = 0 for an
all-zero block).  The output is sum_t P8_t V8_t / sum_t p_t in fp64.

e4m3 (OCP FP8): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; normal
values 2^(E-7) (1 + M/8), subnormals 2^-6 (M/8); largest finite 448; values
are rounded to nearest, ties to even.
"""

import math

import numpy as np

from . import isa_oracle as orc

E4M3_MAX = 448.0


def e4m3_round(x):
    """x rounded to the nearest e4m3 value (ties to even), saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # spacing of the e4m3 grid around |x|: 2^(floor(log2|x|) - 3) for normals,
    # 2^-9 in the subnormal range (|x| < 2^-6)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ex = np.maximum(ex, -6.0)
    step = np.exp2(ex - 3.0)
    q = a / step
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1))
    r = r + up
    return np.sign(x) * np.minimum(r * step, E4M3_MAX)


def block_exponent(amax):
    """Smallest integer e with amax / 2^e <= 448 (0 for amax = 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.zeros(amax.shape)
    nz = amax > 0
    e = np.ceil(np.log2(amax[nz] / E4M3_MAX))
    # guard the ceil against log2 rounding: step to the smallest valid e
    e = np.where(amax[nz] / np.exp2(e - 1) <= E4M3_MAX, e - 1, e)
    e = np.where(amax[nz] / np.exp2(e) > E4M3_MAX, e + 1, e)
    out[nz] = e
    return out


def quantize_rows(X, block=32):
    """Rows of X rounded to e4m3 under one power-of-two scale per `block`
    consecutive columns; returns the dequantised values."""
    X = np.asarray(X, dtype=np.float64)
    n, d = X.shape
    Xb = X.reshape(n, d // block, block)
    e = block_exponent(np.abs(Xb).max(axis=2))
    s = np.exp2(e)[:, :, None]
    return (e4m3_round(Xb / s) * s).reshape(n, d)


def fp8_full_attention_rows(q, Kt, Vt, parts=("q", "k", "v", "p")):
    """The full route of rows q over the key list (Kt, Vt) with the operands
    named in `parts` rounded to e4m3 (the others exact).  The V scale blocks
    are 32 consecutive keys from the start of the list; a short last block is
    padded with zero rows that take no part."""
    d = q.shape[1]
    n = Kt.shape[0]
    pad = (-n) % 32
    q8 = quantize_rows(q) if "q" in parts else np.asarray(q, np.float64)
    k8 = quantize_rows(Kt) if "k" in parts else np.asarray(Kt, np.float64)
    if "v" in parts:
        v8 = quantize_rows(np.concatenate([Vt, np.zeros((pad, Vt.shape[1]))]).T).T[:n]
    else:
        v8 = np.asarray(Vt, np.float64)
    x = (q8 @ k8.T) / math.sqrt(d) / math.log(2.0)   # logits in the exp2 domain
    m = np.ceil(x.max(axis=1, keepdims=True))
    p = np.exp2(x - m)
    p8 = e4m3_round(p) if "p" in parts else p
    return (p8 @ v8) / p.sum(axis=1, keepdims=True)


def error_budget(q, Kt, Vt):
    """Relative L2 error of the full route against exact attention with each
    operand set in e4m3: the evaluation of the FP8 variant."""
    exact = orc.full_attention_rows(q, Kt, Vt)
    norm = np.linalg.norm(exact)
    out = {}
    for name, parts in (("q,k", ("q", "k")), ("v", ("v",)), ("p", ("p",)), ("p,v", ("p", "v")),
                        ("q,k,p,v", ("q", "k", "p", "v"))):
        out[name] = float(np.linalg.norm(fp8_full_attention_rows(q, Kt, Vt, parts) - exact) / norm)
    return out


def main():
    """Error budget of the FP8 full route on the benchmark's input
    distribution (seeded N(0,1) rows, 20 % of the queries sharpened)."""
    from sparse_attention_context_amd.synth import make_inputs
    Q, K, V = make_inputs(1, 2, 128, 2048, 2048, seed=7, dtype="bf16")
    for h in range(2):
        rows = np.arange(0, 2048, 8)
        print("head %d:" % h, {k: round(v, 4) for k, v in error_budget(Q[0, h, rows], K[0, h], V[0, h]).items()})


if __name__ == "__main__":
    main()
