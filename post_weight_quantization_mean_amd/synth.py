"""Seeded synthetic layer inputs (activations X and weights W) for the AWQ scale search.

This module only draws random numbers and rounds them to the storage dtype; it holds none
of the quantization method's arithmetic.  Both the CPU oracle (through the tests) and the
HIP path take their inputs from here, so the two sides see bit-identical data.

Workloads stand in for the calibration activations and trained weights that the pages
measure on (real-model calibration tokens, WikiText-2 evaluation); none of that data is
used.  Recipe, per layer:

* channel magnitudes c_j ~ LogNormal(0, 0.5), j < K;
* n_out outlier channels (drawn without replacement) multiplied by a constant or by
  U(lo, hi) each;
* X entries: ``sign``  -> X[m,j] = +-c_j with a fair random sign (fp32);
             ``gauss`` -> X[m,j] = c_j * g, g ~ N(0,1);
             ``sparse``-> as gauss, then each entry with probability 0.7 is scaled by 0.01
                          (post-activation rows with most entries near zero);
* W entries ~ N(0, 1/K), generated directly in [N, K] (PyTorch Linear.weight) orientation;
  the entries are iid, so this equals the transpose of a K x N draw in distribution.

Random streams: numpy ``Generator(PCG64(SeedSequence([seed, cfg_id, tensor_id])))`` with
tensor_id = 2*layer for X and 2*layer+1 for W.  bf16 tensors are rounded from fp32 with
round-to-nearest-even by torch's CPU cast.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    M: int  # tokens
    K: int  # input channels
    N: int  # output channels (rows of W in [N, K] layout)
    x_kind: str  # "sign" | "gauss" | "sparse"
    n_out: int  # outlier channels
    out_mult: Tuple  # ("const", c) or ("uniform", lo, hi)
    dtype: str  # "f32" | "bf16"


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    name: str
    cfg_id: int
    layers: Tuple[LayerSpec, ...]


def _pct(K: int) -> int:
    return int(round(0.01 * K))


CONFIGS: Dict[str, ConfigSpec] = {
    # Tiny layer: fp32, 3 outlier channels x20, sign-random entries.
    "tiny": ConfigSpec("tiny", 0, (
        LayerSpec("tiny", 64, 256, 128, "sign", 3, ("const", 20.0), "f32"),)),
    # Attention-projection-shaped layer (the headline workload).
    "attn": ConfigSpec("attn", 1, (
        LayerSpec("attn", 4096, 4096, 4096, "gauss", _pct(4096), ("uniform", 10.0, 50.0), "bf16"),)),
    # MLP down-projection-shaped layer: post-activation input, 70% of entries near zero.
    "down": ConfigSpec("down", 2, (
        LayerSpec("down", 4096, 11008, 4096, "sparse", _pct(11008), ("const", 30.0), "bf16"),)),
    # Fused gate+up projection sharing one scale vector: N = 2 x 13824.
    "gate_up": ConfigSpec("gate_up", 3, (
        LayerSpec("gate_up", 8192, 5120, 27648, "gauss", _pct(5120), ("uniform", 10.0, 50.0), "bf16"),)),
    # 8B-style decoder block searched layer by layer; q,k,v share one scale vector (N=6144),
    # gate,up share one (N=28672).
    "block": ConfigSpec("block", 4, (
        LayerSpec("qkv", 16384, 4096, 6144, "gauss", _pct(4096), ("uniform", 10.0, 50.0), "bf16"),
        LayerSpec("o_proj", 16384, 4096, 4096, "gauss", _pct(4096), ("uniform", 10.0, 50.0), "bf16"),
        LayerSpec("gate_up", 16384, 4096, 28672, "gauss", _pct(4096), ("uniform", 10.0, 50.0), "bf16"),
        LayerSpec("down", 16384, 14336, 4096, "sparse", _pct(14336), ("const", 30.0), "bf16"),
    )),
}


def _rng(seed: int, cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, tensor_id])))


def channel_magnitudes(spec: LayerSpec, rng: np.random.Generator) -> np.ndarray:
    c = rng.lognormal(0.0, 0.5, size=spec.K)
    idx = rng.choice(spec.K, size=spec.n_out, replace=False)
    if spec.out_mult[0] == "const":
        c[idx] *= spec.out_mult[1]
    else:
        c[idx] *= rng.uniform(spec.out_mult[1], spec.out_mult[2], size=spec.n_out)
    return c.astype(np.float32)


def _to_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if dtype == "f32" else t.to(torch.bfloat16)


def make_x(spec: LayerSpec, seed: int, cfg_id: int, layer_idx: int, rows: int | None = None) -> torch.Tensor:
    """Activations X [M, K] (CPU tensor, fp32 or bf16).  ``rows`` draws only the first rows
    of the same stream (used for bounded samples); the channel magnitudes are unchanged."""
    rng = _rng(seed, cfg_id, 2 * layer_idx)
    c = channel_magnitudes(spec, rng)
    M = spec.M if rows is None else rows
    if spec.x_kind == "sign":
        sign = rng.integers(0, 2, size=(M, spec.K), dtype=np.int8)
        x = np.where(sign == 1, c[None, :], -c[None, :]).astype(np.float32)
    else:
        x = rng.standard_normal(size=(M, spec.K), dtype=np.float32)
        x *= c[None, :]
        if spec.x_kind == "sparse":
            near_zero = rng.random(size=(M, spec.K), dtype=np.float32) < np.float32(0.7)
            x[near_zero] *= np.float32(0.01)
    return _to_storage(x, spec.dtype)


def make_w(spec: LayerSpec, seed: int, cfg_id: int, layer_idx: int, rows: int | None = None) -> torch.Tensor:
    """Weights W [N, K] (CPU tensor), entries N(0, 1/K).  ``rows`` draws the first rows only."""
    rng = _rng(seed, cfg_id, 2 * layer_idx + 1)
    N = spec.N if rows is None else rows
    w = rng.standard_normal(size=(N, spec.K), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(spec.K))
    return _to_storage(w, spec.dtype)


def make_layer(config: str, layer: int = 0, seed: int = 0) -> Tuple[LayerSpec, torch.Tensor, torch.Tensor]:
    cfg = CONFIGS[config]
    spec = cfg.layers[layer]
    return spec, make_x(spec, seed, cfg.cfg_id, layer), make_w(spec, seed, cfg.cfg_id, layer)


def custom_layer(M: int, K: int, N: int, dtype: str = "bf16", x_kind: str = "gauss", seed: int = 0,
                 n_out: int | None = None, out_mult=("uniform", 10.0, 50.0), cfg_id: int = 100
                 ) -> Tuple[LayerSpec, torch.Tensor, torch.Tensor]:
    """A layer of any shape drawn with the same recipe (ragged-tile and edge-case tests)."""
    spec = LayerSpec("custom", M, K, N, x_kind, _pct(K) if n_out is None else n_out, out_mult, dtype)
    return spec, make_x(spec, seed, cfg_id, 0), make_w(spec, seed, cfg_id, 0)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a CPU fp32/bf16 tensor (both embed exactly in float64)."""
    return t.to(torch.float64).numpy()


def to_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of a CPU fp32/bf16 tensor."""
    return t.to(torch.float32).numpy()


def all_layers() -> List[Tuple[str, int]]:
    return [(c, i) for c, cfg in CONFIGS.items() for i in range(len(cfg.layers))]


def make_layer_device(spec: LayerSpec, device, seed: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """The same recipe drawn with torch's generator on ``device`` (fast for the full-size
    benchmark layers, whose timing does not depend on the values).  The values differ from
    make_x / make_w: this stream is not the numpy one, so parity tests use the CPU generator."""
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * seed + 7919 * spec.K + spec.N)
    c = torch.exp(0.5 * torch.randn(spec.K, generator=g, device=device))
    idx = torch.randperm(spec.K, generator=g, device=device)[:spec.n_out]
    if spec.out_mult[0] == "const":
        c[idx] *= spec.out_mult[1]
    else:
        lo, hi = spec.out_mult[1], spec.out_mult[2]
        c[idx] *= lo + (hi - lo) * torch.rand(spec.n_out, generator=g, device=device)
    if spec.x_kind == "sign":
        x = torch.where(torch.rand((spec.M, spec.K), generator=g, device=device) < 0.5, -c, c)
    else:
        x = torch.randn((spec.M, spec.K), generator=g, device=device) * c
        if spec.x_kind == "sparse":
            x = torch.where(torch.rand((spec.M, spec.K), generator=g, device=device) < 0.7, 0.01 * x, x)
    w = torch.randn((spec.N, spec.K), generator=g, device=device) * (1.0 / spec.K ** 0.5)
    dt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    return x.to(dt), w.to(dt)
