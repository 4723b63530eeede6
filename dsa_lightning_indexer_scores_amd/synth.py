"""Seeded synthetic inputs for the indexer / top-k / sparse-attention stack.

This module only draws random tensors and encodes them in the storage
formats the path consumes (bf16, OCP e4m3fn bytes, fp32).  It holds none of
the method's arithmetic: no scoring, no selection, no attention.  Both the
GPU path's tests and the CPU oracle's tests take their inputs from here, so
the two sides always see the same bytes.

Workloads (sizes as the pages' DSA discussion uses them: a 32K-token
prefill stack with one indexer kept per four layers, a 64K-context decode,
a 128K-token prefill chunked in 4096-query tiles):

  tiny       B=1, L=512, 4 layers 'FSSS', H_I=4, d_I=32, k=64, H=4, d=64,
             bf16 integers uniform in [-3, 3], w uniform in {0,1,2,3}
  pair8k     B=1, L=8192, 'FS', H_I=64, d_I=128 bf16, k=2048, H=16, d=128,
             N(0,1)/sqrt(dim) values, w ~ U(0,1)
  stack32k   B=1, L=32768, 16 layers 'FSSS'x4, indexer e4m3, k=2048,
             H=16, d=128; N(0,1) values, w ~ U(0,1)
  decode64k  B=32, 65536 cached tokens, 24 layers 'FSSS'x6, 64 steps,
             indexer e4m3, k=2048, H=16, d=128; N(0,1), w ~ U(0,1)
  long128k   B=1, L=131072, 8 layers 'FSSSSSSS', indexer e4m3, k=2048,
             chunk 4096 queries; N(0,1), w ~ U(0,1)

Seeds: seed = 1000*config_id + 16*layer + tensor_id (+ 100003*(step+1) for
the per-step decode queries), tensor ids q_I=0, w=1, k_I=2, q=3, kv=4.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import torch

T_QI, T_W, T_KI, T_Q, T_KV = 0, 1, 2, 3, 4
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    B: int
    L: int              # prefill length, or cached context N for decode
    pattern: str
    H_I: int
    d_I: int
    k: int
    H: int
    d: int
    idx_dtype: str      # "bf16" or "fp8"
    dist: str           # "int3", "gauss_scaled" or "gauss"
    chunk: int = 4096
    decode_steps: int = 0

    @property
    def n_layers(self) -> int:
        return len(self.pattern)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 0, 1, 512, "FSSS", 4, 32, 64, 4, 64, "bf16", "int3", 512),
    "pair8k": Workload("pair8k", 1, 1, 8192, "FS", 64, 128, 2048, 16, 128, "bf16", "gauss_scaled", 4096),
    "stack32k": Workload("stack32k", 2, 1, 32768, "FSSS" * 4, 64, 128, 2048, 16, 128, "fp8", "gauss", 4096),
    "decode64k": Workload("decode64k", 3, 32, 65536, "FSSS" * 6, 64, 128, 2048, 16, 128, "fp8", "gauss", 4096, 64),
    "long128k": Workload("long128k", 4, 1, 131072, "FSSSSSSS", 64, 128, 2048, 16, 128, "fp8", "gauss", 4096),
}


def seed_for(cfg: Workload, layer: int, tensor_id: int, step: int = -1) -> int:
    s = 1000 * cfg.config_id + 16 * layer + tensor_id
    if step >= 0:
        s += 100003 * (step + 1)
    return s


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _values(shape, dist: str, dim: int, seed: int, device) -> torch.Tensor:
    """fp32 values of the requested distribution (before storage encoding)."""
    g = _gen(seed, device)
    if dist == "int3":
        return torch.randint(-3, 4, shape, generator=g, device=device).to(torch.float32)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if dist == "gauss_scaled":
        x = x / math.sqrt(dim)
    return x


def encode(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Store fp32 values as bf16 (RNE) or OCP e4m3fn bytes (RNE, clamped to +-448).

    e4m3 data is returned as a uint8 tensor of codes, the form the C ABI takes.
    """
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "fp8":
        return x.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    raise ValueError(dtype)


def weights(shape, dist: str, seed: int, device) -> torch.Tensor:
    g = _gen(seed, device)
    if dist == "int3":
        return torch.randint(0, 4, shape, generator=g, device=device).to(torch.float32)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def prefill_layer(cfg: Workload, layer: int, device="cpu", L: Optional[int] = None,
                  B: Optional[int] = None, with_indexer: Optional[bool] = None) -> Dict[str, torch.Tensor]:
    """Inputs of one layer of a prefill stack.

    Returns q [B,L,H,d] bf16 and kv [B,L,2,d] bf16 (row = K then V) for every
    layer, plus q_I [B,L,H_I,d_I], w [B,L,H_I] fp32 and k_I [B,L,d_I] for
    layers that run the indexer ('F').  q_I / k_I are bf16 or e4m3 codes.
    """
    L = cfg.L if L is None else L
    B = cfg.B if B is None else B
    if with_indexer is None:
        with_indexer = cfg.pattern[layer] in "F1"
    out = {}
    if with_indexer:
        out["q_I"] = encode(_values((B, L, cfg.H_I, cfg.d_I), cfg.dist, cfg.d_I,
                                    seed_for(cfg, layer, T_QI), device), cfg.idx_dtype)
        out["w"] = weights((B, L, cfg.H_I), cfg.dist, seed_for(cfg, layer, T_W), device)
        out["k_I"] = encode(_values((B, L, cfg.d_I), cfg.dist, cfg.d_I,
                                    seed_for(cfg, layer, T_KI), device), cfg.idx_dtype)
    out["q"] = encode(_values((B, L, cfg.H, cfg.d), cfg.dist, cfg.d,
                              seed_for(cfg, layer, T_Q), device), "bf16")
    out["kv"] = encode(_values((B, L, 2, cfg.d), cfg.dist, cfg.d,
                               seed_for(cfg, layer, T_KV), device), "bf16")
    return out


def prefill_stack(cfg: Workload, device="cpu", L: Optional[int] = None, B: Optional[int] = None,
                  pattern: Optional[str] = None) -> List[Dict[str, torch.Tensor]]:
    pattern = cfg.pattern if pattern is None else pattern
    return [prefill_layer(cfg, i, device, L, B, with_indexer=(c in "F1"))
            for i, c in enumerate(pattern)]


def decode_caches(cfg: Workload, device="cuda", N: Optional[int] = None, B: Optional[int] = None,
                  steps: Optional[int] = None, pattern: Optional[str] = None) -> List[Dict[str, torch.Tensor]]:
    """Per-layer caches with capacity N + steps rows: k_I [B,cap,d_I] (F layers) and kv [B,cap,2,d].

    Rows N..N+steps-1 hold the tokens that the decode steps append (the
    caller's write of the new row is this pre-drawn row becoming visible).
    """
    N = cfg.L if N is None else N
    B = cfg.B if B is None else B
    steps = cfg.decode_steps if steps is None else steps
    pattern = cfg.pattern if pattern is None else pattern
    cap = N + steps
    layers = []
    for i, c in enumerate(pattern):
        lay = {}
        if c in "F1":
            lay["k_I"] = decode_k_I(cfg, i, device, N, B, steps)
        lay["kv"] = encode(_values((B, cap, 2, cfg.d), cfg.dist, cfg.d,
                                   seed_for(cfg, i, T_KV), device), "bf16")
        layers.append(lay)
    return layers


def decode_k_I(cfg: Workload, layer: int, device="cuda", N: Optional[int] = None, B: Optional[int] = None,
               steps: Optional[int] = None) -> torch.Tensor:
    """The indexer key cache k_I [B, N + steps, d_I] of one layer (its seeds do not depend on
    whether the pattern makes the layer F, so a layer's keys are the same in every pattern)."""
    N = cfg.L if N is None else N
    B = cfg.B if B is None else B
    steps = cfg.decode_steps if steps is None else steps
    return encode(_values((B, N + steps, cfg.d_I), cfg.dist, cfg.d_I, seed_for(cfg, layer, T_KI), device),
                  cfg.idx_dtype)


def decode_queries(cfg: Workload, step: int, device="cuda", B: Optional[int] = None,
                   pattern: Optional[str] = None) -> List[Dict[str, torch.Tensor]]:
    """The new token's queries at one decode step: q_I [B,1,H_I,d_I], w [B,1,H_I] (F layers), q [B,1,H,d]."""
    B = cfg.B if B is None else B
    pattern = cfg.pattern if pattern is None else pattern
    layers = []
    for i, c in enumerate(pattern):
        lay = {}
        if c in "F1":
            lay["q_I"] = encode(_values((B, 1, cfg.H_I, cfg.d_I), cfg.dist, cfg.d_I,
                                        seed_for(cfg, i, T_QI, step), device), cfg.idx_dtype)
            lay["w"] = weights((B, 1, cfg.H_I), cfg.dist, seed_for(cfg, i, T_W, step), device)
        lay["q"] = encode(_values((B, 1, cfg.H, cfg.d), cfg.dist, cfg.d,
                                  seed_for(cfg, i, T_Q, step), device), "bf16")
        layers.append(lay)
    return layers


def ragged_stack(cfg: Workload, n_seq: int = 64, q_new: int = 512, Lk: int = 8192, seed: int = 77,
                 device="cuda"):
    """The ragged prefill workload: n_seq sequences each bring q_new queries continuing a cached
    prefix of 0 .. Lk - q_new tokens (uniform), through cfg's pattern with cfg's layer shapes.
    Queries are packed over the sequences ([T, ...], T = n_seq * q_new) and caches are per
    sequence ([n_seq, Lk, ...]).  N(0,1) values, w ~ U(0,1), e4m3 indexer inputs.
    Returns (layers, q_len, pos0)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    q_len = [q_new] * n_seq
    pos0 = [int(x) for x in rng.integers(0, Lk - q_new + 1, size=n_seq)]
    T = n_seq * q_new
    g = torch.Generator(device=device).manual_seed(seed)
    layers = []
    for c in cfg.pattern:
        lay = {"q": torch.randn((T, cfg.H, cfg.d), generator=g, device=device).to(torch.bfloat16),
               "kv": torch.randn((n_seq, Lk, 2, cfg.d), generator=g, device=device).to(torch.bfloat16)}
        if c in "F1":
            lay["q_I"] = encode(torch.randn((T, cfg.H_I, cfg.d_I), generator=g, device=device), "fp8")
            lay["w"] = torch.rand((T, cfg.H_I), generator=g, device=device)
            lay["k_I"] = encode(torch.randn((n_seq, Lk, cfg.d_I), generator=g, device=device), "fp8")
        layers.append(lay)
    return layers, q_len, pos0


def bits_u16(x: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (raw storage, no conversion)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def bits_u8(x: torch.Tensor):
    """e4m3 code tensor (uint8) -> numpy uint8 codes."""
    return x.detach().cpu().contiguous().view(torch.uint8).numpy()


def raw(x: torch.Tensor):
    """Raw storage of an input tensor as numpy, for the oracle to decode itself."""
    if x.dtype == torch.bfloat16:
        return bits_u16(x)
    if x.dtype == torch.uint8:
        return bits_u8(x)
    return x.detach().cpu().contiguous().numpy()
