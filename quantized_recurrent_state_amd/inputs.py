"""Seeded synthetic inputs and the workload table.

This module holds no arithmetic of the method: it only draws the per-step
inputs q, k, v, alpha, beta with the shapes and distributions of the pages'
workloads, and lists the workloads.  Both the HIP path and the CPU oracle are
fed from the same tensors it returns.

Distributions follow the synthetic stand-ins for the pages' trained models
(Gated DeltaNet 0.8B on held-out articles, natural text to 32K — "When Dynamic
Scaling Fails", project page; the families of the LinQuant summary's Eq. (1)
and of the "Preserving Updates" abstract).  N(mu, x) is read with x as the
variance.  Every step's inputs are drawn from a generator seeded by
(seed, layer, step), so a step's inputs do not depend on how steps are
chunked.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# numeric values of the library's enumerations
POLICY_NONE, POLICY_DYNAMIC, POLICY_PERSISTENT, POLICY_YOKED = 0, 1, 2, 3
ROUND_RNE, ROUND_BDR, ROUND_DITHER, ROUND_BDR_A, ROUND_BDR_B = 0, 1, 2, 3, 4
DECAY_SCALAR, DECAY_DIAG = 0, 1

RECIPES = ("la", "gla", "gdn", "mamba2")


def _mix(seed: int, layer: int, step: int) -> int:
    """Deterministic 63-bit seed for one (seed, layer, step)."""
    x = (seed * 0x9E3779B97F4A7C15 + layer * 0xBF58476D1CE4E5B9 + step * 0x94D049BB133111EB + 1)
    x &= (1 << 64) - 1
    x ^= x >> 31
    x = (x * 0xD6E8FEB86659FD93) & ((1 << 64) - 1)
    x ^= x >> 29
    return x & ((1 << 63) - 1)


def outlier_channels(seed: int, dk: int, count: int = 2) -> list[int]:
    """Two distinct key channels, drawn once from the seed (CPU generator)."""
    g = torch.Generator(device="cpu").manual_seed(_mix(seed, 0x5EED, 0))
    return sorted(torch.randperm(dk, generator=g)[:count].tolist())


def _normal(shape, g, device, mean=0.0, var=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if var != 1.0:
        x = x * (var ** 0.5)
    if mean != 0.0:
        x = x + mean
    return x


def _l2n(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def gen_step(recipe: str, n: int, dk: int, dv: int, seed: int, layer: int, step: int,
             device="cpu", outliers: list[int] | None = None) -> dict:
    """Inputs of one step for n heads: q,k [n,Dk]; v [n,Dv]; alpha [n] or [n,Dk]; beta [n]."""
    g = torch.Generator(device=device).manual_seed(_mix(seed, layer, step))
    if recipe == "la":          # linear attention, scalar decay
        q = _l2n(_normal((n, dk), g, device))
        k = _l2n(_normal((n, dk), g, device))
        v = _normal((n, dv), g, device)
        alpha = torch.sigmoid(_normal((n,), g, device, 3.0, 0.5))
        beta = torch.sigmoid(_normal((n,), g, device))
    elif recipe == "gla":       # diagonal decay, two outlier key channels x8
        q = _l2n(_normal((n, dk), g, device))
        k = _normal((n, dk), g, device)
        if outliers:
            k[:, outliers] *= 8.0
        k = _l2n(k)
        v = _normal((n, dv), g, device)
        # exp(-softplus(x)) written as sigmoid(-x)
        alpha = torch.sigmoid(-_normal((n, dk), g, device, -3.0, 1.0))
        beta = torch.sigmoid(_normal((n,), g, device))
    elif recipe == "gdn":       # gated delta rule, scalar gate
        q = _l2n(_normal((n, dk), g, device))
        k = _l2n(_normal((n, dk), g, device))
        v = _normal((n, dv), g, device)
        alpha = torch.sigmoid(_normal((n,), g, device, 4.0, 0.5))
        beta = torch.sigmoid(_normal((n,), g, device))
    elif recipe == "mamba2":    # SSM-style scalar decay, unnormalised keys
        q = _normal((n, dk), g, device, 0.0, 1.0 / dk)
        k = _normal((n, dk), g, device, 0.0, 1.0 / dk)
        v = _normal((n, dv), g, device)
        alpha = torch.exp(-0.1 * torch.nn.functional.softplus(_normal((n,), g, device, -2.0, 1.0)))
        beta = torch.nn.functional.softplus(_normal((n,), g, device))
    else:
        raise ValueError(f"unknown input recipe {recipe!r}")
    return {"q": q.contiguous(), "k": k.contiguous(), "v": v.contiguous(),
            "alpha": alpha.contiguous(), "beta": beta.contiguous()}


def gen_steps(recipe: str, n_per_layer: int, dk: int, dv: int, seeds, t0: int, steps: int,
              device="cpu", out: dict | None = None) -> dict:
    """Inputs of steps [t0, t0+steps) for len(seeds) layers of n_per_layer heads each
    (layer-major along the head axis).  Tensors carry a leading [steps] axis.
    ``out`` may hold preallocated tensors to fill."""
    seeds = list(seeds)
    n = n_per_layer * len(seeds)
    outl = outlier_channels(seeds[0], dk) if recipe == "gla" else None
    diag = recipe == "gla"
    if out is None:
        out = {"q": torch.empty((steps, n, dk), device=device),
               "k": torch.empty((steps, n, dk), device=device),
               "v": torch.empty((steps, n, dv), device=device),
               "alpha": torch.empty((steps, n, dk) if diag else (steps, n), device=device),
               "beta": torch.empty((steps, n), device=device)}
    for t in range(steps):
        for li, sd in enumerate(seeds):
            d = gen_step(recipe, n_per_layer, dk, dv, sd, 0, t0 + t, device, outl)
            sl = slice(li * n_per_layer, (li + 1) * n_per_layer)
            for key in out:
                out[key][t, sl] = d[key]
    return out


@dataclass(frozen=True)
class Arm:
    """One handle's configuration inside a workload."""
    name: str
    bits: int
    group: int
    policy: int
    rounding: int
    layers: tuple = (0,)   # layer indices folded into the batch; seeds are per layer
    lrb_rank: int = 0      # Low-Rank Bypass slots (0: off)
    scale_fmt: int = 0     # stored group-scale format: 0 fp32, 1 binary16, 2 bfloat16


@dataclass(frozen=True)
class Workload:
    """A synthetic workload: shape, input recipe, horizon and its arms."""
    name: str
    recipe: str
    batch: int          # per layer
    heads: int
    dk: int
    dv: int
    delta: int
    decay: int
    steps: int          # decode horizon H
    warmup: int         # fp32 warmup steps before persistent calibration (0: start at S_0 = 0)
    arms: tuple = field(default_factory=tuple)
    shared_inputs: bool = True   # arms run on identical inputs (comparison arms)

    def arm_config(self, arm: Arm) -> dict:
        return dict(batch=self.batch * len(arm.layers), heads=self.heads, dk=self.dk, dv=self.dv,
                    bits=arm.bits, group=arm.group, policy=arm.policy, rounding=arm.rounding,
                    delta=self.delta, decay=self.decay, lrb_rank=arm.lrb_rank,
                    scale_fmt=arm.scale_fmt)


WORKLOADS = {
    # linear attention, scalar decay, delta = 0
    "la": Workload("la-1x1-64x64-int8g64-dynamic-rne", "la", 1, 1, 64, 64, 0, DECAY_SCALAR,
                   256, 0, (Arm("int8g64-dynamic", 8, 64, POLICY_DYNAMIC, ROUND_RNE),)),
    # GLA-style diagonal decay, delta = 0, persistent INT4 after a 64-step fp32 warmup
    "gla": Workload("gla-64x16-128x128-int4g32-persistent-rne", "gla", 64, 16, 128, 128, 0,
                    DECAY_DIAG, 1024, 64,
                    (Arm("int4g32-persistent", 4, 32, POLICY_PERSISTENT, ROUND_RNE),)),
    # Gated DeltaNet, delta = 1: dynamic vs yoked scale on identical inputs
    "gdn": Workload("gdn-256x16-128x128-int4g32-dynamic-vs-yoked", "gdn", 256, 16, 128, 128, 1,
                    DECAY_SCALAR, 2048, 0,
                    (Arm("int4g32-dynamic", 4, 32, POLICY_DYNAMIC, ROUND_RNE),
                     Arm("int4g32-yoked", 4, 32, POLICY_YOKED, ROUND_RNE))),
    # Mamba-2-style scalar decay, delta = 0, Dv = 64: BDR vs RNE on identical inputs
    "mamba2": Workload("mamba2-128x64-64x128-int8g64-persistent-bdr-vs-rne", "mamba2", 128, 64,
                       128, 64, 0, DECAY_SCALAR, 4096, 64,
                       (Arm("int8g64-persistent-bdr", 8, 64, POLICY_PERSISTENT, ROUND_BDR),
                        Arm("int8g64-persistent-rne", 8, 64, POLICY_PERSISTENT, ROUND_RNE))),
    # 24 independent Gated DeltaNet layers x batch 512 x 32 heads; layers 0-3 INT8 g64,
    # layers 4-23 INT4 g32; persistent scale; BDR; inputs seeded per layer
    "stack24": Workload("gdn24-512x32-128x128-mixed-int8g64-int4g32-persistent-bdr", "gdn", 512,
                        32, 128, 128, 1, DECAY_SCALAR, 32768, 64,
                        (Arm("layers0-3-int8g64", 8, 64, POLICY_PERSISTENT, ROUND_BDR,
                             tuple(range(0, 4))),
                         Arm("layers4-23-int4g32", 4, 32, POLICY_PERSISTENT, ROUND_BDR,
                             tuple(range(4, 24)))),
                        shared_inputs=False),
}


def _stack24_variant(key: str, name: str, rounding: int, int4_group: int,
                     lrb_rank: int = 0, scale_fmt: int = 0, int8_group: int = 64) -> Workload:
    base = WORKLOADS["stack24"]
    gname = lambda g: f"g{g}" if g else "head"       # group 0: one scale per head
    return Workload(name, base.recipe, base.batch, base.heads, base.dk, base.dv, base.delta,
                    base.decay, base.steps, base.warmup,
                    (Arm(f"layers0-3-int8{gname(int8_group)}", 8, int8_group, POLICY_PERSISTENT,
                         rounding, tuple(range(0, 4)), lrb_rank, scale_fmt),
                     Arm(f"layers4-23-int4{gname(int4_group)}", 4, int4_group, POLICY_PERSISTENT,
                         rounding, tuple(range(4, 24)), lrb_rank, scale_fmt)),
                    shared_inputs=False)


# The same stack with the other roundings, and with 16-element INT4 groups
# (INT4 + one fp32 scale per 16 elements: 6 bits per element, 5.33x below fp32).
WORKLOADS["stack24-rne"] = _stack24_variant(
    "stack24-rne", "gdn24-512x32-128x128-mixed-int8g64-int4g32-persistent-rne", ROUND_RNE, 32)
WORKLOADS["stack24-dither"] = _stack24_variant(
    "stack24-dither", "gdn24-512x32-128x128-mixed-int8g64-int4g32-persistent-dither", ROUND_DITHER, 32)
WORKLOADS["stack24-g16"] = _stack24_variant(
    "stack24-g16", "gdn24-512x32-128x128-mixed-int8g64-int4g16-persistent-bdr", ROUND_BDR, 16)
# ... with bfloat16 group scales (INT4 g32: 4.5 bits per element), and with INT4 g16 and
# bfloat16 scales (5 bits per element)
WORKLOADS["stack24-bf16"] = _stack24_variant(
    "stack24-bf16", "gdn24-512x32-128x128-mixed-int8g64-int4g32-bf16scale-persistent-bdr", ROUND_BDR,
    32, scale_fmt=2)
WORKLOADS["stack24-g16-bf16"] = _stack24_variant(
    "stack24-g16-bf16", "gdn24-512x32-128x128-mixed-int8g64-int4g16-bf16scale-persistent-bdr",
    ROUND_BDR, 16, scale_fmt=2)
# Gated DeltaNet with a dynamic scale per head (group 0): every row updated before any is
# requantised (two passes over the head's rows)
WORKLOADS["gdn-head"] = Workload("gdn-256x16-128x128-int4-headscale-dynamic", "gdn", 256, 16, 128, 128,
                                 1, DECAY_SCALAR, 2048, 0,
                                 (Arm("int4head-dynamic", 4, 0, POLICY_DYNAMIC, ROUND_RNE),))
# ... with one scale per head (group 0) instead of group scales
WORKLOADS["stack24-head"] = _stack24_variant(
    "stack24-head", "gdn24-512x32-128x128-mixed-int8-int4-headscale-persistent-bdr", ROUND_BDR, 0,
    int8_group=0)
# ... with the directional-rounding reading B' (sensitivity flag)
WORKLOADS["stack24-bdrb"] = _stack24_variant(
    "stack24-bdrb", "gdn24-512x32-128x128-mixed-int8g64-int4g32-persistent-bdr-reading-b", ROUND_BDR_B, 32)
# ... and with a rank-4 Low-Rank Bypass in every layer
WORKLOADS["stack24-lrb4"] = _stack24_variant(
    "stack24-lrb4", "gdn24-512x32-128x128-mixed-int8g64-int4g32-persistent-bdr-lrb4", ROUND_BDR, 32,
    lrb_rank=4)


@dataclass(frozen=True)
class PrefillWorkload:
    """A synthetic chunkwise-prefill workload: T prompt tokens into every head's state."""
    name: str
    recipe: str
    batch: int
    heads: int
    dk: int
    dv: int
    decay: int
    tokens: int
    bits: int
    group: int
    policy: int

    def config(self) -> dict:
        return dict(batch=self.batch, heads=self.heads, dk=self.dk, dv=self.dv, bits=self.bits,
                    group=self.group, policy=self.policy, rounding=ROUND_RNE, delta=0,
                    decay=self.decay)


PREFILL_WORKLOADS = {
    # GLA-style diagonal decay (the linear write the chunkwise form covers): a 4096-token
    # prompt into batch 64 x 16 heads of INT4 g32 state, dynamic scale from S_0 = 0
    "prefill-gla": PrefillWorkload("gla-prefill-64x16-128x128-int4g32-dynamic-T4096", "gla", 64, 16,
                                   128, 128, DECAY_DIAG, 4096, 4, 32, POLICY_DYNAMIC),
}
