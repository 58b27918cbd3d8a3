"""Seeded synthetic inputs for the dropless MoE layer.

This module is the only code shared by the CPU oracle and the HIP path's tests.
It draws random numbers and rounds them to the storage precision of a run; it
holds none of the layer's arithmetic (no routing, no GEMM, no activation).

Workloads follow the pages' layers: Qwen3-30B-A3B and Qwen3-235B-A22B MoE layers
with 128 experts and top-8 random routing (Prime Mega MoE write-ups, single-layer
table: "1 node, 8xH200, EP=8, 128 experts, top-8, random routing").  Hidden sizes
are not on the pages; they come from the public Qwen3 model shapes
(H=2048/I=768 and H=4096/I=1536).

Streams (numpy PCG64 through ``SeedSequence(seed).spawn(9)``; child i does not depend
on how many are spawned): 0 logits, 1 x, 2 W_gate, 3 W_up, 4 W_down, 5 dY, 6 skew
permutation, 7 Gumbel noise, 8 router weight W_r (N(0,1)/sqrt(H), [H, E]).
x and dY are N(0,1); W_gate/W_up are N(0,1)/sqrt(H); W_down is N(0,1)/sqrt(I);
logits are N(0,1) fp32, or Zipf-biased Gumbel logits for the skewed workload.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

__all__ = ["MoeConfig", "CONFIGS", "make_inputs", "make_router_weight", "bf16_round", "bf16_bits", "bits_to_f32"]


@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int            # tokens
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # routed experts
    k: int            # experts per token
    e_begin: int      # first local expert
    e_local: int      # number of local experts
    seed: int
    dtype: str = "bf16"      # "bf16" or "f32": x, weights, dY
    bwd: str = "bf16"        # "bf16" or "mxfp8" backward GEMMs
    fwd: str = "bf16"        # "bf16" or "mxfp8" forward GEMMs
    routing: str = "gauss"   # "gauss": N(0,1) logits; "zipf": biased Gumbel logits
    renorm: int = 1          # 1: softmax over the k selected logits; 0: over all E
    row_tile: int = 0        # rows per tile of the bf16 row-tiled GEMMs: 0 chosen by the library, 256, 320

    def replace(self, **kw) -> "MoeConfig":
        return dataclasses.replace(self, **kw)

    @property
    def R_cap(self) -> int:
        return self.T * min(self.k, self.e_local)


CONFIGS = {
    # tiny layer: T64 H128 I64 E8 top-2, in fp32 and in bf16
    "tiny_f32": MoeConfig("tiny_f32", 64, 128, 64, 8, 2, 0, 8, 0, dtype="f32"),
    "tiny_bf16": MoeConfig("tiny_bf16", 64, 128, 64, 8, 2, 0, 8, 0),
    # Qwen3-30B-A3B-shaped layer, all 128 experts on one GPU
    "qwen3_30b": MoeConfig("qwen3_30b", 4096, 2048, 768, 128, 8, 0, 128, 1),
    # Qwen3-235B-A22B-shaped layer, one GPU's EP=8 share (experts 0..15 of 128)
    "qwen3_235b_ep8": MoeConfig("qwen3_235b_ep8", 16384, 4096, 1536, 128, 8, 0, 16, 2),
    # skewed dropless routing at the 30B shape: Zipf(1.2) expert loads, 8 experts empty
    "skew_zipf": MoeConfig("skew_zipf", 16384, 2048, 768, 128, 8, 0, 128, 3, routing="zipf"),
    # the 235B share with an MXFP8 backward
    "qwen3_235b_ep8_fp8bwd": MoeConfig("qwen3_235b_ep8_fp8bwd", 16384, 4096, 1536, 128, 8, 0, 16, 2,
                                       bwd="mxfp8"),
    # the pages' mxfp8 mode (MXFP8 forward and backward GEMMs) at both layer shapes
    "qwen3_235b_ep8_mxfp8": MoeConfig("qwen3_235b_ep8_mxfp8", 16384, 4096, 1536, 128, 8, 0, 16, 2,
                                      bwd="mxfp8", fwd="mxfp8"),
    "qwen3_30b_mxfp8": MoeConfig("qwen3_30b_mxfp8", 4096, 2048, 768, 128, 8, 0, 128, 1, bwd="mxfp8", fwd="mxfp8"),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exact fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    return bits_to_f32(bf16_bits(x))


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def _zipf_logits(cfg: MoeConfig, rng_perm, rng_gumbel) -> np.ndarray:
    """Gumbel-perturbed log-Zipf(1.2) biases: top-k of these logits draws each token's
    expert set without replacement with weights rank^-1.2; the 8 lowest ranks get a
    bias of -1e4 and never win, so they receive no tokens."""
    E = cfg.E
    ranks = rng_perm.permutation(E) + 1          # rank of expert e, 1..E
    bias = np.where(ranks <= E - 8, -1.2 * np.log(ranks.astype(np.float64)), -1e4)
    g = rng_gumbel.gumbel(size=(cfg.T, E))
    return (bias[None, :] + g).astype(np.float32)


def make_inputs(cfg: MoeConfig, with_weights: bool = True, with_dy: bool = True) -> dict:
    """All inputs of one fwd+bwd pass of ``cfg``.

    Float tensors are returned as fp32 arrays whose values are exactly representable
    in the run's storage dtype (bf16 rounding, RNE, when ``cfg.dtype == 'bf16'``).
    Weights are the local slice [e_local, ...].  Logits are always fp32.
    """
    ss = np.random.SeedSequence(cfg.seed).spawn(8)
    rng = [np.random.Generator(np.random.PCG64(s)) for s in ss]
    out = {}
    if cfg.routing == "gauss":
        out["logits"] = _normal(rng[0], (cfg.T, cfg.E))
    elif cfg.routing == "zipf":
        out["logits"] = _zipf_logits(cfg, rng[6], rng[7])
    else:
        raise ValueError(cfg.routing)
    rnd = bf16_round if cfg.dtype == "bf16" else (lambda a: a)
    out["x"] = rnd(_normal(rng[1], (cfg.T, cfg.H)))
    if with_weights:
        El, H, I = cfg.e_local, cfg.H, cfg.I
        out["w_gate"] = rnd(_normal(rng[2], (El, H, I), 1.0 / np.sqrt(H)))
        out["w_up"] = rnd(_normal(rng[3], (El, H, I), 1.0 / np.sqrt(H)))
        out["w_down"] = rnd(_normal(rng[4], (El, I, H), 1.0 / np.sqrt(I)))
    if with_dy:
        out["dy"] = rnd(_normal(rng[5], (cfg.T, cfg.H)))
    return out


def make_router_weight(cfg: MoeConfig) -> np.ndarray:
    """Router weight W_r [H, E] of ``cfg`` (all E experts), rounded like the other inputs."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(cfg.seed).spawn(9)[8]))
    w = _normal(rng, (cfg.H, cfg.E), 1.0 / np.sqrt(cfg.H))
    return bf16_round(w) if cfg.dtype == "bf16" else w
