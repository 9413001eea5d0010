"""Seeded synthetic KV caches for tests and benchmarks.

This module only makes inputs: it holds none of the coding arithmetic (no
model, no coder, no calibration), and both the CPU oracle's tests and the HIP
path's tests and benchmark draw their inputs from it.

The stand-in workload.  The pages measure real Qwen3 KV caches (0.6B to 32B
targets, FP8 predictor, held-out C4, sigma and p_hat calibrated on 128
examples; "Speculative KV coding", section "早期结果" (early results)).
Neither the weights nor the data are available, so a generator with the same
cache geometry stands in for them:

* per-channel scale s_c = exp(0.5 N(0,1)) for every (layer, kv, head, dim),
  with two outlier channels (chosen by the model seed) scaled by 20;
* x = bf16(s_c * N(0,1));
* residual r drawn per scalar from 95% N(0,1), 3% N(0,9) (std 3) and 2%
  Student-t with 3 degrees of freedom (unscaled);
* mu = x + sigma_c * r with sigma_c = k * s_c, rounded to the predictor
  format (bf16, or kept fp32);
* FP8 caches code e4m3(x) (round to nearest even, saturating at +-448).

A drifting variant stands in for caches whose local statistics change along
the sequence, the case the online-entropy-estimation page builds its adaptive
counts for: each (layer, kv, head) row's scale is multiplied by
exp(sin(2 pi t / 2048 + phi)), phi uniform per row, so the row's values and
its residuals grow and shrink together over the tokens (about 2.7x either
way), while sigma and p_hat are calibrated once, on sequences with their own
phases.

A second kind of predictor stands in for the FP8 model's own cache ("同一模型
的优化版本": the predictor is a quantized copy of the same model): mu is the
block-FP8 round trip of x itself, with one fp32 scale per 32 consecutive
channels of a token (amax / 448), so the residual is bounded, structured
rounding noise rather than the mixture above.

Layout of x and mu: [layers][2 (K, V)][kv_heads][tokens][head_dim].
Symbols are returned as raw bit patterns (uint16 for bf16, uint8 for e4m3);
bf16 predictor means as uint16 bit patterns, fp32 ones as float32.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

SYM_BF16, SYM_E4M3 = 0, 1
MU_BF16, MU_F32 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # 1..5, used for seeds
    layers: int
    kv_heads: int
    head_dim: int
    tokens: int
    sym_fmt: int
    mu_fmt: int
    sigma_k: float        # sigma_c = sigma_k * s_c
    calib_seqs: int
    calib_tokens: int
    mu_kind: str = "mixture"  # "mixture": x + sigma_c r; "fp8block": block-FP8 round trip of x;
                              # "drift": the mixture with a scale that drifts along tokens
    sigma_mode: int = 0       # how the coder resolves sigma: 0 per channel, 1 per channel and |mu| octave
    phat_mode: int = 0        # p_hat: 0 the calibrated histogram, 1 adaptive (decayed counts per chunk)

    @property
    def model_seed(self) -> int:
        return 1000 + self.index

    @property
    def data_seed(self) -> int:
        return 2000 + self.index

    def calib_seed(self, j: int) -> int:
        return 3000 + 1000 * self.index + j

    @property
    def n_scalars(self) -> int:
        return self.layers * 2 * self.kv_heads * self.tokens * self.head_dim

    @property
    def n_channels(self) -> int:
        return self.layers * 2 * self.kv_heads * self.head_dim

    @property
    def sym_bytes(self) -> int:
        return 2 if self.sym_fmt == SYM_BF16 else 1

    @property
    def mu_bytes(self) -> int:
        return 2 if self.mu_fmt == MU_BF16 else 4

    def with_tokens(self, tokens: int, layers: int | None = None, name: str | None = None) -> "Workload":
        return Workload(name or self.name, self.index, layers or self.layers, self.kv_heads, self.head_dim,
                        tokens, self.sym_fmt, self.mu_fmt, self.sigma_k, self.calib_seqs, self.calib_tokens,
                        self.mu_kind, self.sigma_mode, self.phat_mode)


WORKLOADS = {
    w.name: w
    for w in [
        # 1 layer, K and V, 2 KV heads, head_dim 64, 256 tokens
        Workload("tiny_bf16", 1, 1, 2, 64, 256, SYM_BF16, MU_BF16, 0.02, 1, 256),
        # Qwen3-0.6B cache geometry: 28 layers x 8 KV heads x 128, 2048 tokens
        Workload("qwen3_0.6b_bf16", 2, 28, 8, 128, 2048, SYM_BF16, MU_BF16, 0.02, 128, 512),
        # same geometry, native FP8 cache at 8192 tokens, fp32 predictor mean
        Workload("qwen3_0.6b_e4m3", 3, 28, 8, 128, 8192, SYM_E4M3, MU_F32, 0.05, 128, 512),
        # Qwen3-32B cache geometry: 64 layers x 8 KV heads x 128, 8192 tokens
        Workload("qwen3_32b_bf16", 4, 64, 8, 128, 8192, SYM_BF16, MU_BF16, 0.015, 128, 512),
        # Qwen3-32B FP8 cache at 32768 tokens, bf16 predictor mean
        Workload("qwen3_32b_e4m3_32k", 5, 64, 8, 128, 32768, SYM_E4M3, MU_BF16, 0.04, 128, 512),
        # Qwen3-32B geometry with an FP8-quantized copy of the cache as the predictor
        Workload("qwen3_32b_bf16_fp8res", 6, 64, 8, 128, 8192, SYM_BF16, MU_BF16, 0.0, 128, 512, "fp8block"),
        # the same data coded with sigma per channel and octave of |mu| (same seeds)
        Workload("qwen3_32b_bf16_fp8res_oct", 6, 64, 8, 128, 8192, SYM_BF16, MU_BF16, 0.0, 128, 512, "fp8block", 1),
        # Qwen3-0.6B FP8 cache geometry whose scale (values and residuals) drifts along tokens
        Workload("qwen3_0.6b_e4m3_drift", 7, 28, 8, 128, 8192, SYM_E4M3, MU_F32, 0.05, 128, 512, "drift"),
        # the same data coded with the adaptive p_hat (same seeds)
        Workload("qwen3_0.6b_e4m3_drift_adapt", 7, 28, 8, 128, 8192, SYM_E4M3, MU_F32, 0.05, 128, 512, "drift", 0, 1),
        # the 32K-token FP8 cache coded with the adaptive p_hat (same seeds as qwen3_32b_e4m3_32k)
        Workload("qwen3_32b_e4m3_32k_adapt", 5, 64, 8, 128, 32768, SYM_E4M3, MU_BF16, 0.04, 128, 512, "mixture", 0, 1),
    ]
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def channel_scales(w: Workload) -> torch.Tensor:
    """s_c for every (layer, kv, head, dim), float32 [L, 2, H, D] on the CPU."""
    g = _gen(w.model_seed, "cpu")
    s = torch.exp(0.5 * torch.randn(w.layers, 2, w.kv_heads, w.head_dim, generator=g, dtype=torch.float64))
    flat = s.view(-1)
    outliers = torch.randperm(flat.numel(), generator=g)[:2]
    flat[outliers] *= 20.0
    return s.to(torch.float32)


def _residual(shape, g, device) -> torch.Tensor:
    u = torch.rand(shape, generator=g, device=device)
    z = torch.randn(shape, generator=g, device=device)
    r = torch.where(u < 0.98, torch.where(u < 0.95, z, 3.0 * z), torch.zeros((), device=device))
    heavy = (u >= 0.98).nonzero(as_tuple=True)
    nh = heavy[0].numel()
    if nh:
        zz = torch.randn(nh, generator=g, device=device)
        chi2 = torch.randn(nh, 3, generator=g, device=device).square().sum(1)
        r[heavy] = zz / torch.sqrt(chi2 / 3.0)
    return r


FP8_BLOCK = 32  # channels per block-FP8 scale


def fp8_block_roundtrip(xf: torch.Tensor) -> torch.Tensor:
    """dequant(e4m3(x / scale)) * scale along the last dim in blocks of 32,
    scale = amax(|x|) / 448 per block (fp32; an all-zero block keeps scale 1)."""
    shp = xf.shape
    xb = xf.reshape(*shp[:-1], shp[-1] // FP8_BLOCK, FP8_BLOCK)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (xb / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float32)
    return (q * scale).reshape(shp)


DRIFT_PERIOD = 2048   # tokens
DRIFT_AMPLITUDE = 1.0  # of the log scale


def _drift(g, kv_heads: int, tokens: int, device) -> torch.Tensor:
    """exp(a sin(2 pi t / P + phi)) per (kv, head) row and token, phi uniform per row."""
    phi = 2.0 * torch.pi * torch.rand(2, kv_heads, 1, 1, generator=g, device=device)
    t = torch.arange(tokens, device=device, dtype=torch.float32).view(1, 1, tokens, 1)
    return torch.exp(DRIFT_AMPLITUDE * torch.sin(2.0 * torch.pi * t / DRIFT_PERIOD + phi))


def _slab(w: Workload, s_layer: torch.Tensor, tokens: int, seed: int, device):
    """One layer: x bits and mu for [2, H, tokens, D]."""
    g = _gen(seed, device)
    shape = (2, w.kv_heads, tokens, w.head_dim)
    sc = s_layer.to(device).view(2, w.kv_heads, 1, w.head_dim)
    if w.mu_kind == "drift":
        # values and residuals scale together with a drift of the (layer, kv, head) row
        sc = sc * _drift(g, w.kv_heads, tokens, device)
    x16 = (sc * torch.randn(shape, generator=g, device=device)).to(torch.bfloat16)
    xf = x16.to(torch.float32)
    if w.mu_kind == "fp8block":
        mu = fp8_block_roundtrip(xf)
    else:
        mu = xf + (w.sigma_k * sc) * _residual(shape, g, device)
    if w.sym_fmt == SYM_BF16:
        xb = x16.view(torch.int16)
    else:
        xb = xf.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    mub = mu.to(torch.bfloat16).view(torch.int16) if w.mu_fmt == MU_BF16 else mu
    return xb, mub


def generate(w: Workload, seed: int | None = None, tokens: int | None = None, device="cpu",
             layers: range | None = None):
    """x (symbol bits) and mu for the workload, [L, 2, H, T, D] on `device`.

    Each layer is drawn from its own stream, so a subset of layers can be made
    alone and matches the same layers of the whole cache on the same device.
    """
    seed = w.data_seed if seed is None else seed
    tokens = w.tokens if tokens is None else tokens
    layers = range(w.layers) if layers is None else layers
    s = channel_scales(w)
    xs, mus = [], []
    for l in layers:
        xb, mub = _slab(w, s[l], tokens, seed * 1_000_003 + l, device)
        xs.append(xb)
        mus.append(mub)
    return torch.stack(xs), torch.stack(mus)


def calibration_set(w: Workload, j: int, device="cpu"):
    """Calibration sequence j (0 <= j < calib_seqs): same model seed, its own data seed."""
    return generate(w, seed=w.calib_seed(j), tokens=w.calib_tokens, device=device)
