"""Seeded synthetic ISA inputs shaped like video-DiT attention latents.

This module holds no arithmetic of the method: it only draws Q, K, V and
shapes them like an in-context editing layer (context keys scaled down, a
fraction of source queries sharpened towards a source key).  Both the HIP
path and the CPU oracle consume what it returns.

Recipe (one numpy PCG64 generator per call, fixed draw order):
  1. Q ~ N(0,1) [B,H,Ns,d]; K ~ N(0,1) and V ~ N(0,1) [B,H,Ns+Nc,d] (float32).
  2. Context keys scaled per clip (consecutive spans of the Nc context rows).
  3. Per (batch, head): perm = permutation(Ns); the first floor(sharp*Ns)
     entries of perm get q += 4 * k_t with t ~ integers(0, Ns) (unscaled
     source keys, drawn with replacement).
  4. bf16 workloads: round to bfloat16, nearest-even (values stay float32
     arrays that are exactly representable in bfloat16).
"""

import numpy as np


def round_to_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def make_inputs(B, H, d, Ns, Nc, seed, dtype="bf16", clips=((1.0, 0.5),), sharp=0.20):
    """Return float32 numpy arrays Q [B,H,Ns,d], K and V [B,H,Ns+Nc,d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Q = rng.standard_normal((B, H, Ns, d), dtype=np.float32)
    K = rng.standard_normal((B, H, Ns + Nc, d), dtype=np.float32)
    V = rng.standard_normal((B, H, Ns + Nc, d), dtype=np.float32)
    lo = 0
    for i, (frac, scale) in enumerate(clips):
        hi = Nc if i == len(clips) - 1 else lo + int(round(frac * Nc))
        K[:, :, Ns + lo:Ns + hi] *= np.float32(scale)
        lo = hi
    nsh = int(np.floor(sharp * Ns))
    for x in range(B):
        for h in range(H):
            perm = rng.permutation(Ns)
            t = rng.integers(0, Ns, nsh) if Ns > 0 else np.zeros(0, dtype=np.int64)
            Q[x, h, perm[:nsh]] += np.float32(4.0) * K[x, h, t]
    if dtype == "bf16":
        Q, K, V = round_to_bf16(Q), round_to_bf16(K), round_to_bf16(V)
    return Q, K, V


def make_inputs_device(B, H, d, Ns, Nc, seed, device, dtype="bf16", clips=((1.0, 0.5),), sharp=0.20):
    """The recipe above drawn on the GPU with torch's generator (seeded), for
    timing runs that do not need the host copy: torch tensors Q [B,H,Ns,d],
    K and V [B,H,Ns+Nc,d] in bf16 (round to nearest even) or float32.  The
    values differ from make_inputs' numpy draw; shapes, distributions and
    structure are the same."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    Q = torch.randn((B, H, Ns, d), generator=g, device=device, dtype=torch.float32)
    K = torch.randn((B, H, Ns + Nc, d), generator=g, device=device, dtype=torch.float32)
    V = torch.randn((B, H, Ns + Nc, d), generator=g, device=device, dtype=torch.float32)
    lo = 0
    for i, (frac, scale) in enumerate(clips):
        hi = Nc if i == len(clips) - 1 else lo + int(round(frac * Nc))
        K[:, :, Ns + lo:Ns + hi] *= scale
        lo = hi
    nsh = int(np.floor(sharp * Ns))
    for x in range(B):
        for h in range(H):
            perm = torch.randperm(Ns, generator=g, device=device)[:nsh]
            t = torch.randint(0, Ns, (nsh,), generator=g, device=device)
            Q[x, h, perm] += 4.0 * K[x, h, t]
    if dtype == "bf16":
        Q, K, V = (t.to(torch.bfloat16) for t in (Q, K, V))
    return Q, K, V


def workload_inputs(w, heads=None):
    """Inputs of a Workload (configs.py).  heads=None draws all w.H heads."""
    H = w.H if heads is None else heads
    return make_inputs(w.B, H, w.d, w.Ns, w.Nc, w.seed, w.dtype, w.clips, w.sharp)


def make_local_inputs(B, H, d, Ns, Nc, b, sigma, seed, sharp=0.2):
    """Inputs with within-block locality, as tokens of neighbouring video
    patches have: each block of b rows (cut per segment from its own start,
    source then context) draws a centre c ~ N(0, I) for K and one for V, and
    every row is sqrt(1 - sigma^2) c + sigma N(0, I).  sigma = 1 is i.i.d.
    rows, sigma -> 0 identical rows in a block.  Q ~ N(0, I), and a fraction
    `sharp` of each head's queries get q += 4 k_t for a random source key t.
    fp64, no rounding (for the CPU diagnostics)."""
    rng = np.random.default_rng(seed)
    a = np.sqrt(max(0.0, 1.0 - sigma * sigma))
    bounds = [(s, min(s + b, Ns)) for s in range(0, Ns, b)] + [(Ns + s, Ns + min(s + b, Nc)) for s in range(0, Nc, b)]
    Q = rng.standard_normal((B, H, Ns, d))
    K = sigma * rng.standard_normal((B, H, Ns + Nc, d))
    V = sigma * rng.standard_normal((B, H, Ns + Nc, d))
    nsh = int(sharp * Ns)
    for x in range(B):
        for h in range(H):
            for s, e in bounds:
                K[x, h, s:e] += a * rng.standard_normal(d)
                V[x, h, s:e] += a * rng.standard_normal(d)
            perm = rng.permutation(Ns)[:nsh]
            Q[x, h, perm] += 4.0 * K[x, h, rng.integers(0, Ns, nsh)]
    return Q, K, V
