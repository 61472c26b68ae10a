"""Seeded synthetic inputs for GDPA (shared by the oracle tests and the HIP path).

This module only draws numbers; it holds none of the method's arithmetic.  Both
the fp64 oracle and the HIP library read what it produces, so that parity is
checked on identical inputs.

The pages measure on internal ads data (Kunlun paper summary, section 4,
"Experimental Results"), which is not public.  The workloads below are synthetic
stand-ins: jagged user-history batches whose long-sequence range matches the
HSP discussion of sequences longer than 1000 events (section 2.2), with per-sample
context-derived K/V (section 2.2, GDPA bullet; Telegram review, layer steps 1-2).

Draw order (per seed): lengths, then Q, then K, then V, then dO.  For the stacked
workload: lengths, X0, C, then per layer W_K, W_V, then dO.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

# numpy draws are made in chunks of this many elements so that the float32
# staging copy stays small; chunked draws give the same stream as one draw.
_CHUNK = 1 << 24


@dataclass(frozen=True)
class GdpaConfig:
    """Shape of one synthetic GDPA workload."""
    name: str
    batch: int
    heads: int
    head_dim: int
    n_kv: int
    lengths: tuple            # ("fixed", L) | ("uniform", lo, hi) | ("lognormal", median, max)
    dtype: str                # "f32" | "bf16"
    phis: tuple               # score maps the workload runs
    backward: bool = False
    layers: int = 0           # >0: stacked residual layers with generated K/V
    ctx_dim: int = 0          # context feature width for weight generation


CONFIGS = {
    1: GdpaConfig("fp32 fixed-length B=4 L=64 H=2 d=32 n=64", 4, 2, 32, 64,
                  ("fixed", 64), "f32", ("softmax", "silu")),
    2: GdpaConfig("bf16 SiLU fwd B=256 L~U[64,1024] H=4 d=64 n=256", 256, 4, 64, 256,
                  ("uniform", 64, 1024), "bf16", ("silu",)),
    3: GdpaConfig("bf16 softmax fwd B=512 L~logN(512,max 4096) H=8 d=128 n=512", 512, 8, 128,
                  512, ("lognormal", 512, 4096), "bf16", ("softmax",)),
    4: GdpaConfig("bf16 fwd+bwd B=256 L~U[256,2048] H=4 d=128 n=1024", 256, 4, 128, 1024,
                  ("uniform", 256, 2048), "bf16", ("softmax", "silu"), backward=True),
    5: GdpaConfig("bf16 stacked 4-layer SiLU fwd+bwd B=1024 L~logN(1024,max 8192) H=8 d=128 "
                  "n=256 ctx=512", 1024, 8, 128, 256, ("lognormal", 1024, 8192), "bf16",
                  ("silu",), backward=True, layers=4, ctx_dim=512),
}


def draw_lengths(rng: np.random.Generator, spec: tuple, batch: int) -> np.ndarray:
    """Per-sample sequence lengths (int64) for one of the three length laws.

    Log-normal: l = round(median * exp(z)), z ~ N(0, 1), accepted when 1 <= l <= max
    (rejection keeps the law truncated, sigma = 1).
    """
    kind = spec[0]
    if kind == "fixed":
        return np.full(batch, int(spec[1]), dtype=np.int64)
    if kind == "uniform":
        lo, hi = int(spec[1]), int(spec[2])
        return rng.integers(lo, hi + 1, batch).astype(np.int64)
    if kind == "lognormal":
        median, mx = float(spec[1]), int(spec[2])
        out = []
        while len(out) < batch:
            l = int(round(median * math.exp(1.0 * rng.standard_normal())))
            if 1 <= l <= mx:
                out.append(l)
        return np.asarray(out, dtype=np.int64)
    if kind == "explicit":
        return np.asarray(spec[1], dtype=np.int64)
    raise ValueError(f"unknown length law {spec!r}")


def offsets_from_lengths(lengths) -> np.ndarray:
    """offsets[B+1] with offsets[0] = 0 and offsets[b+1] - offsets[b] = lengths[b]."""
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def _torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def draw_normal(rng: np.random.Generator, shape, dtype: str, divisor: float = 1.0) -> torch.Tensor:
    """N(0,1) float32 draws divided by `divisor`, stored as `dtype` (bf16 rounds to nearest even)."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=_torch_dtype(dtype))
    pos = 0
    while pos < n:
        m = min(_CHUNK, n - pos)
        x = rng.standard_normal(m, dtype=np.float32)
        if divisor != 1.0:
            x /= np.float32(divisor)
        out[pos:pos + m] = torch.from_numpy(x).to(out.dtype)
        pos += m
    return out.view(*shape)


def draw_uniform(rng: np.random.Generator, shape, dtype: str, bound: float) -> torch.Tensor:
    """U(-bound, bound) from float32 uniforms on [0, 1), stored as `dtype`."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=_torch_dtype(dtype))
    pos = 0
    b = np.float32(bound)
    while pos < n:
        m = min(_CHUNK, n - pos)
        x = rng.random(m, dtype=np.float32)
        x = (x * np.float32(2.0) - np.float32(1.0)) * b
        out[pos:pos + m] = torch.from_numpy(x).to(out.dtype)
        pos += m
    return out.view(*shape)


@dataclass
class GdpaInputs:
    """One drawn GDPA problem: host tensors in the library's layouts.

    q, do: [T, H, d]; k, v: [B, n, H, d]; offsets: int32 [B+1].
    """
    cfg: GdpaConfig
    lengths: np.ndarray
    offsets: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: Optional[torch.Tensor] = None

    @property
    def total_tokens(self) -> int:
        return int(self.offsets[-1])


def make_gdpa_inputs(cfg: GdpaConfig, seed: int = 0, sharp: bool = False,
                     with_grad: Optional[bool] = None) -> GdpaInputs:
    """Draw lengths, Q, K, V (and dO when the workload has a backward pass).

    Values ~ N(0,1)/sqrt(d).  `sharp=True` draws Q and K as N(0,1) instead, which
    makes the scores ~N(0,1) so that softmax is far from uniform.
    """
    rng = np.random.default_rng(seed)
    lengths = draw_lengths(rng, cfg.lengths, cfg.batch)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    H, d, n, B = cfg.heads, cfg.head_dim, cfg.n_kv, cfg.batch
    qk_div = 1.0 if sharp else math.sqrt(d)
    q = draw_normal(rng, (T, H, d), cfg.dtype, qk_div)
    k = draw_normal(rng, (B, n, H, d), cfg.dtype, qk_div)
    v = draw_normal(rng, (B, n, H, d), cfg.dtype, math.sqrt(d))
    if with_grad is None:
        with_grad = cfg.backward
    do = draw_normal(rng, (T, H, d), cfg.dtype) if with_grad else None
    return GdpaInputs(cfg, lengths, torch.from_numpy(off.astype(np.int32)), q, k, v, do)


@dataclass
class StackedInputs:
    """Stacked residual GDPA workload with generated K/V.

    x0, do: [T, H*d]; ctx: [B, ctx_dim]; w_k[l], w_v[l]: [n*H*d, ctx_dim] (output-major).
    """
    cfg: GdpaConfig
    lengths: np.ndarray
    offsets: torch.Tensor
    x0: torch.Tensor
    ctx: torch.Tensor
    w_k: list = field(default_factory=list)
    w_v: list = field(default_factory=list)
    do: Optional[torch.Tensor] = None


def xavier_uniform_bound(fan_in: int, fan_out: int) -> float:
    return math.sqrt(6.0 / (fan_in + fan_out))


def make_stacked_inputs(cfg: GdpaConfig, seed: int = 0) -> StackedInputs:
    """Draw the stacked workload: lengths, X0 ~ N(0,1)/sqrt(d), C ~ N(0,1),
    per layer W_K, W_V ~ Xavier-uniform(fan_in=ctx_dim, fan_out=n*H*d), then dO ~ N(0,1)."""
    assert cfg.layers > 0 and cfg.ctx_dim > 0
    rng = np.random.default_rng(seed)
    lengths = draw_lengths(rng, cfg.lengths, cfg.batch)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    H, d, n, B, C = cfg.heads, cfg.head_dim, cfg.n_kv, cfg.batch, cfg.ctx_dim
    x0 = draw_normal(rng, (T, H * d), cfg.dtype, math.sqrt(d))
    ctx = draw_normal(rng, (B, C), cfg.dtype)
    a = xavier_uniform_bound(C, n * H * d)
    w_k, w_v = [], []
    for _ in range(cfg.layers):
        w_k.append(draw_uniform(rng, (n * H * d, C), cfg.dtype, a))
        w_v.append(draw_uniform(rng, (n * H * d, C), cfg.dtype, a))
    do = draw_normal(rng, (T, H * d), cfg.dtype)
    return StackedInputs(cfg, lengths, torch.from_numpy(off.astype(np.int32)), x0, ctx, w_k, w_v, do)


def small_config(base: GdpaConfig, **kw) -> GdpaConfig:
    """A copy of `base` with some fields replaced (used to shrink workloads for tests)."""
    return replace(base, **kw)


@dataclass
class SwaInputs:
    """Sliding-window self-attention inputs: Q, K, V, dO all [T, H, d] from the sequence."""
    lengths: np.ndarray
    offsets: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor

    @property
    def total_tokens(self) -> int:
        return int(self.offsets[-1])


def make_swa_inputs(length_spec: tuple, batch: int, H: int, d: int, seed: int = 0,
                    sharp: bool = False, dtype: str = "bf16") -> SwaInputs:
    """Draw lengths, then Q, K, V ~ N(0,1)/sqrt(d) (Q and K ~ N(0,1) when sharp), then
    dO ~ N(0,1), all [T, H, d] and rounded to `dtype`."""
    rng = np.random.default_rng(seed)
    lengths = draw_lengths(rng, length_spec, batch)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    qk_div = 1.0 if sharp else math.sqrt(d)
    q = draw_normal(rng, (T, H, d), dtype, qk_div)
    k = draw_normal(rng, (T, H, d), dtype, qk_div)
    v = draw_normal(rng, (T, H, d), dtype, math.sqrt(d))
    do = draw_normal(rng, (T, H, d), dtype)
    return SwaInputs(lengths, torch.from_numpy(off.astype(np.int32)), q, k, v, do)


@dataclass
class PmaInputs:
    """Seed pooling inputs: seeds [m,H,d]; K, V [T,H,d] from the sequence; dO [B,m,H,d]."""
    lengths: np.ndarray
    offsets: torch.Tensor
    seeds: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor

    @property
    def total_tokens(self) -> int:
        return int(self.offsets[-1])


def make_pma_inputs(length_spec: tuple, batch: int, H: int, d: int, m: int, seed: int = 0,
                    sharp: bool = False, dtype: str = "bf16") -> PmaInputs:
    """Draw lengths, then seeds [m,H,d] and K [T,H,d] ~ N(0,1)/sqrt(d) (N(0,1) when sharp),
    then V ~ N(0,1)/sqrt(d), then dO [B,m,H,d] ~ N(0,1), all rounded to `dtype`."""
    rng = np.random.default_rng(seed)
    lengths = draw_lengths(rng, length_spec, batch)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    qk_div = 1.0 if sharp else math.sqrt(d)
    seeds = draw_normal(rng, (m, H, d), dtype, qk_div)
    k = draw_normal(rng, (T, H, d), dtype, qk_div)
    v = draw_normal(rng, (T, H, d), dtype, math.sqrt(d))
    do = draw_normal(rng, (batch, m, H, d), dtype)
    return PmaInputs(lengths, torch.from_numpy(off.astype(np.int32)), seeds, k, v, do)


@dataclass
class JaggedKvInputs:
    """GDPA inputs with a jagged context: K, V [rows,H,d], sample b owning rows kv_offsets[b]:kv_offsets[b+1]."""
    lengths: np.ndarray
    kv_counts: np.ndarray
    offsets: torch.Tensor
    kv_offsets: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor

    @property
    def n_kv(self) -> int:
        return int(self.kv_counts.max())


def make_jagged_kv_inputs(length_spec: tuple, count_spec: tuple, batch: int, H: int, d: int,
                          seed: int = 0, sharp: bool = False, dtype: str = "bf16") -> JaggedKvInputs:
    """Draw token lengths, then context row counts (each >= 1), then Q, K, V ~ N(0,1)/sqrt(d)
    (Q and K ~ N(0,1) when sharp), then dO ~ N(0,1), rounded to `dtype`."""
    rng = np.random.default_rng(seed)
    lengths = draw_lengths(rng, length_spec, batch)
    counts = np.maximum(draw_lengths(rng, count_spec, batch), 1)
    off = offsets_from_lengths(lengths)
    kv_off = offsets_from_lengths(counts)
    T, N = int(off[-1]), int(kv_off[-1])
    qk_div = 1.0 if sharp else math.sqrt(d)
    q = draw_normal(rng, (T, H, d), dtype, qk_div)
    k = draw_normal(rng, (N, H, d), dtype, qk_div)
    v = draw_normal(rng, (N, H, d), dtype, math.sqrt(d))
    do = draw_normal(rng, (T, H, d), dtype)
    return JaggedKvInputs(lengths, counts, torch.from_numpy(off.astype(np.int32)),
                          torch.from_numpy(kv_off.astype(np.int32)), q, k, v, do)


@dataclass
class LayerStackInputs:
    """Inputs of the Kunlun layer stack: token states X0 [T,H,d], context C [B,c], per-layer
    weight-generation matrices W_K, W_V [n*H*d, c], pooling seeds [m,H,d], upstream gradients."""
    lengths: np.ndarray
    offsets: torch.Tensor
    x0: torch.Tensor
    ctx: torch.Tensor
    w_k: list
    w_v: list
    seeds: list
    dx: torch.Tensor
    dz: list


def make_layer_stack_inputs(length_spec: tuple, batch: int, H: int, d: int, n: int, ctx_dim: int,
                            layers: int, m: int, seed: int = 0) -> LayerStackInputs:
    """Draw lengths, X0 ~ N(0,1)/sqrt(d), C ~ N(0,1), then per layer W_K, W_V ~ U(+-xavier) and
    seeds ~ N(0,1)/sqrt(d), then dX ~ N(0,1) [T,H,d] and per layer dZ ~ N(0,1) [B,m,H,d]; bf16."""
    rng = np.random.default_rng(seed)
    lengths = draw_lengths(rng, length_spec, batch)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    x0 = draw_normal(rng, (T, H, d), "bf16", math.sqrt(d))
    ctx = draw_normal(rng, (batch, ctx_dim), "bf16")
    bound = xavier_uniform_bound(ctx_dim, n * H * d)
    w_k, w_v, seeds = [], [], []
    for _ in range(layers):
        w_k.append(draw_uniform(rng, (n * H * d, ctx_dim), "bf16", bound))
        w_v.append(draw_uniform(rng, (n * H * d, ctx_dim), "bf16", bound))
        seeds.append(draw_normal(rng, (m, H, d), "bf16", math.sqrt(d)))
    dx = draw_normal(rng, (T, H, d), "bf16")
    dz = [draw_normal(rng, (batch, m, H, d), "bf16") for _ in range(layers)]
    return LayerStackInputs(lengths, torch.from_numpy(off.astype(np.int32)), x0, ctx, w_k, w_v, seeds, dx, dz)


def draw_ffn_biases(seed: int, bias_rows_shape, B: int, H: int, d: int, out_scale: Optional[float] = None):
    """FFN biases as float32: a score bias shaped `bias_rows_shape` ([B,n,H] dense or
    [rows,H] jagged), N(0,1) like the scores, and an output bias [B,H,d], N(0,1) *
    out_scale (default 1/sqrt(d), the scale of the V rows the output mixes)."""
    rng = np.random.default_rng(seed)
    sb = draw_normal(rng, tuple(bias_rows_shape), "f32")
    ob = draw_normal(rng, (B, H, d), "f32") * (1.0 / math.sqrt(d) if out_scale is None else out_scale)
    return sb, ob


# Event-level personalisation: one GDPA problem per event type over the same
# users, with sizes that follow the event's value (larger head width, more heads
# and more context rows for the valuable, rarer events; a narrow, long sequence
# for the plentiful low-value one).  The pages name the knobs, not their values:
# these sizes are a synthetic reading.
EVENT_TYPES = {
    "click": GdpaConfig("click B=256 L~U[64,1024] H=8 d=128 n=512", 256, 8, 128, 512,
                        ("uniform", 64, 1024), "bf16", ("silu",), backward=True),
    "impression": GdpaConfig("impression B=256 L~U[256,2048] H=4 d=64 n=128", 256, 4, 64, 128,
                             ("uniform", 256, 2048), "bf16", ("silu",), backward=True),
    "conversion": GdpaConfig("conversion B=256 L~U[16,256] H=8 d=128 n=256", 256, 8, 128, 256,
                             ("uniform", 16, 256), "bf16", ("silu",), backward=True),
}


def make_event_inputs(seed: int = 0, shrink: int = 1, sharp: bool = False):
    """{event type: GdpaInputs} for EVENT_TYPES; shrink > 1 divides the batch and
    the sequence lengths (small parity cases of the same mix)."""
    out = {}
    for i, (name, cfg) in enumerate(EVENT_TYPES.items()):
        if shrink > 1:
            kind, lo, hi = cfg.lengths
            cfg = small_config(cfg, batch=max(cfg.batch // shrink, 2),
                               lengths=(kind, max(lo // shrink, 1), max(hi // shrink, 2)))
        out[name] = make_gdpa_inputs(cfg, seed=seed + 101 * i, sharp=sharp)
    return out
