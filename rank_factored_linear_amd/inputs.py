"""Seeded synthetic inputs for the theta-bundle projection.

This module only draws numbers: it holds none of the method's arithmetic (no
band map, no decomposition, no projection).  Both the HIP path and the float64
oracle are fed from here, and each consumes the exact stored values it draws.

The recipes follow the five workloads the library is measured on: Gemma-shaped
layer stacks with the value distributions named below.  N(0, sd) means a
normal distribution with standard deviation ``sd``; U(a, b) is uniform.

Seeds are ``SeedSequence([2026, workload, layer, family, tensor])``; the same
key drives NumPy on the host and a torch Philox generator on the device.
"""

from __future__ import annotations

import numpy as np

FAMILIES = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")

# (out_dim, in_dim) of each family.
SHAPES_26 = {  # 26-layer stack, hidden 1152, MLP width 6912
    "q_proj": (1024, 1152), "k_proj": (256, 1152), "v_proj": (256, 1152), "o_proj": (1152, 1024),
    "gate_proj": (6912, 1152), "up_proj": (6912, 1152), "down_proj": (1152, 6912),
}
SHAPES_60 = {  # 60-layer stack, hidden 5376, MLP width 21504
    "q_proj": (8192, 5376), "k_proj": (2048, 5376), "v_proj": (2048, 5376), "o_proj": (5376, 8192),
    "gate_proj": (21504, 5376), "up_proj": (21504, 5376), "down_proj": (5376, 21504),
}

# Tensor ids inside a seed key.
T_W, T_W0, T_S, T_U, T_V, T_X, T_A, T_NOISE, T_B, T_P, T_Q = range(11)

# Tiny fp32 stack: 4 layers in the two bands [0, 1] and [2, 3] as the workload
# states them; one projection out=256, in=512.
TINY_LAYERS = 4
TINY_LAYER_BAND = (0, 0, 1, 1)
TINY_OUT, TINY_IN, TINY_TOKENS = 256, 512, 8


def seed_key(workload: int, layer: int, family: int, tensor: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([2026, workload, layer, family, tensor])


def rng(workload: int, layer: int, family: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_key(workload, layer, family, tensor)))


def torch_seed(workload: int, layer: int, family: int, tensor: int) -> int:
    st = seed_key(workload, layer, family, tensor).generate_state(2, np.uint32)
    return (int(st[0]) << 31) ^ int(st[1])


def fam_id(family: str) -> int:
    return FAMILIES.index(family)


# ---------------------------------------------------------------------------
# bfloat16 storage (round to nearest even), done once at input creation.
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16 (nearest, ties to even); 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Host draws
# ---------------------------------------------------------------------------


def normal(shape, sd: float, key: tuple) -> np.ndarray:
    return (rng(*key).standard_normal(shape, dtype=np.float32) * np.float32(sd)).astype(np.float32)


def uniform(shape, lo: float, hi: float, key: tuple) -> np.ndarray:
    return rng(*key).uniform(lo, hi, size=shape).astype(np.float32)


def normal_bf16(shape, sd: float, key: tuple) -> np.ndarray:
    return f32_to_bf16_bits(normal(shape, sd, key))


def uniform_bf16(shape, lo: float, hi: float, key: tuple) -> np.ndarray:
    return f32_to_bf16_bits(uniform(shape, lo, hi, key))


# Workload 1: tiny fp32 stack ------------------------------------------------


def tiny_stack(seed_workload: int = 1):
    """Per-layer weights W_l = a_l B_band + P_l Q_l^T + N(0, 1e-3), in float64.

    B_band ~ N(0, 0.02) [256, 512] per band, a_l ~ U(0.8, 1.2), P_l [256, 8] and
    Q_l [512, 8] ~ N(0, 0.05), and x ~ N(0, 1) [8, 512].  The band of each
    layer is the literal list of the workload, not a computed map.
    """
    w = seed_workload
    B = [rng(w, b, 0, T_B).normal(0.0, 0.02, (TINY_OUT, TINY_IN)) for b in range(2)]
    weights = []
    for l in range(TINY_LAYERS):
        a = rng(w, l, 0, T_A).uniform(0.8, 1.2)
        P = rng(w, l, 0, T_P).normal(0.0, 0.05, (TINY_OUT, 8))
        Q = rng(w, l, 0, T_Q).normal(0.0, 0.05, (TINY_IN, 8))
        noise = rng(w, l, 0, T_NOISE).normal(0.0, 1e-3, (TINY_OUT, TINY_IN))
        weights.append(a * B[TINY_LAYER_BAND[l]] + P @ Q.T + noise)
    x = rng(w, 0, 0, T_X).normal(0.0, 1.0, (TINY_TOKENS, TINY_IN))
    return weights, x


# Workloads 2-4: bf16 bundles -------------------------------------------------


def bundle_bf16_host(workload: int, family: str, shapes: dict, layer: int, band: int, rank: int,
                     passthrough: bool = False):
    """One (layer, family) bundle as bf16 bit patterns, drawn on the host.

    W0 ~ N(0, 0.02) is keyed by band (one block per band and family).  With
    ``passthrough`` s = 1 exactly and rank is 0; otherwise s ~ U(0.9, 1.1) and
    U, V ~ N(0, 0.01).
    """
    out_dim, in_dim = shapes[family]
    f = fam_id(family)
    w0 = normal_bf16((out_dim, in_dim), 0.02, (workload, band, f, T_W0))
    if passthrough:
        s = f32_to_bf16_bits(np.ones(out_dim, np.float32))
    else:
        s = uniform_bf16((out_dim,), 0.9, 1.1, (workload, layer, f, T_S))
    u = normal_bf16((out_dim, rank), 0.01, (workload, layer, f, T_U))
    v = normal_bf16((in_dim, rank), 0.01, (workload, layer, f, T_V))
    return {"W0": w0, "s": s, "U": u, "V": v}


def activations_bf16_host(workload: int, family: str, shapes: dict, layer: int, tokens: int):
    _, in_dim = shapes[family]
    return normal_bf16((tokens, in_dim), 1.0, (workload, layer, fam_id(family), T_X))


# ---------------------------------------------------------------------------
# Device draws (large stacks): torch's Philox generator keyed like the host.
# ---------------------------------------------------------------------------


def device_normal(torch, shape, sd: float, key: tuple, device, dtype):
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(*key))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(sd)
    return t.to(dtype)


def device_uniform(torch, shape, lo: float, hi: float, key: tuple, device, dtype):
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(*key))
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(hi - lo).add_(lo)
    return t.to(dtype)


def device_bundle(torch, workload: int, family: str, shapes: dict, layer: int, band: int, rank: int,
                  device="cuda", dtype=None, with_w0: bool = True):
    """One (layer, family) bundle drawn on the device (bf16 by default)."""
    dtype = dtype or torch.bfloat16
    out_dim, in_dim = shapes[family]
    f = fam_id(family)
    out = {}
    if with_w0:
        out["W0"] = device_normal(torch, (out_dim, in_dim), 0.02, (workload, band, f, T_W0), device, dtype)
    out["s"] = device_uniform(torch, (out_dim,), 0.9, 1.1, (workload, layer, f, T_S), device, dtype)
    out["U"] = device_normal(torch, (out_dim, rank), 0.01, (workload, layer, f, T_U), device, dtype)
    out["V"] = device_normal(torch, (in_dim, rank), 0.01, (workload, layer, f, T_V), device, dtype)
    return out


def device_w0(torch, workload: int, family: str, shapes: dict, band: int, device="cuda", dtype=None):
    dtype = dtype or torch.bfloat16
    out_dim, in_dim = shapes[family]
    return device_normal(torch, (out_dim, in_dim), 0.02, (workload, band, fam_id(family), T_W0), device, dtype)


def device_activations(torch, workload: int, family: str, shapes: dict, layer: int, tokens: int,
                       device="cuda", dtype=None):
    dtype = dtype or torch.bfloat16
    _, in_dim = shapes[family]
    return device_normal(torch, (tokens, in_dim), 1.0, (workload, layer, fam_id(family), T_X), device, dtype)


def device_original(torch, w0_bf16, workload: int, family: str, layer: int, device="cuda"):
    """Original fp32 weight a * W0_band + N(0, 2e-3), a ~ U(0.95, 1.05) per (layer, family).

    ``w0_bf16`` is the band's stored block; the caller picks the band.
    """
    f = fam_id(family)
    a = float(rng(workload, layer, f, T_A).uniform(0.95, 1.05))
    noise = device_normal(torch, tuple(w0_bf16.shape), 2e-3, (workload, layer, f, T_NOISE), device, torch.float32)
    return noise.add_(w0_bf16.float(), alpha=a)
