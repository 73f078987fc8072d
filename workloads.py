"""Seeded synthetic workloads for one DP rank's sharded Adam step.

This module holds the five workload definitions (parameter lists, bucket
size, DP size D, ranks, Adam hyper-parameters, value distributions) and the
seeded generators of their inputs. It is the one module that both sides use:
the HIP path's tests and bench.py, and the oracle's tests. It holds none of
the step's arithmetic: bf16 values are made by torch's own fp32 -> bf16
conversion of normal draws, and every random number the step consumes is an
input here.

Seeds follow one rule, seed(cfg, step, role, j) = 0x5EED*10**6 + cfg*10**5 +
step*10**3 + role*100 + j, so any tensor of any workload can be regenerated
alone. Draws use torch.Generator on the device the tensor is made on (CPU:
Mersenne twister, GPU: Philox); the two devices give different values for
one seed, which is fine because the oracle always reads back the bytes that
the device under test received.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 0x5EED * 10**6
ROLES = {"grad": 1, "master": 2, "m": 3, "v": 4, "param": 5, "probe": 6, "sizes": 7, "perm": 8}

# Chunk (elements) for device-side generation, so that the fp32 temporary of
# a 2.2e9-element slice stays at 1 GiB.
_GEN_CHUNK = 1 << 28


def seed(cfg: int, step: int, role: str, j: int = 0) -> int:
    if not (0 <= j < 100 and 0 <= step < 100):
        raise ValueError("seed: j and step must be in [0, 100)")
    return SEED_BASE + cfg * 10**5 + step * 10**3 + ROLES[role] * 100 + j


# ----------------------------------------------------------------------------
# Parameter lists (model-definition order).
# ----------------------------------------------------------------------------

def gpt2_small_params() -> list[int]:
    """GPT-2 small: token and position embeddings, 12 blocks, final LN; the LM
    head is tied to the token embedding. 148 tensors, 124,439,808 elements."""
    h, vocab, ctx, layers = 768, 50257, 1024, 12
    sizes = [vocab * h, ctx * h]
    for _ in range(layers):
        sizes += [h, h,                 # ln_1 weight, bias
                  h * 3 * h, 3 * h,     # attn.c_attn weight, bias
                  h * h, h,             # attn.c_proj weight, bias
                  h, h,                 # ln_2 weight, bias
                  h * 4 * h, 4 * h,     # mlp.c_fc weight, bias
                  4 * h * h, h]         # mlp.c_proj weight, bias
    sizes += [h, h]                     # ln_f weight, bias
    return sizes


def llama3_params(hidden: int, layers: int, ffn: int, kv_heads: int, vocab: int,
                  head_dim: int = 128) -> list[int]:
    """Llama-3 layout: embedding, per layer [input norm, q, k, v, o, post-attention
    norm, gate, up, down], final norm, untied LM head."""
    kv = kv_heads * head_dim
    sizes = [vocab * hidden]
    for _ in range(layers):
        sizes += [hidden, hidden * hidden, hidden * kv, hidden * kv, hidden * hidden,
                  hidden, hidden * ffn, hidden * ffn, ffn * hidden]
    sizes += [hidden, vocab * hidden]
    return sizes


def frag_params() -> list[int]:
    """20,000 sizes log-uniform on [1, 4096] (floor(exp(U ln 4097)), U ~ U[0,1))
    plus 64 tensors of 1,048,576, in a seeded random order."""
    rng = np.random.Generator(np.random.PCG64(seed(5, 0, "sizes")))
    u = rng.random(20000)
    small = np.floor(np.exp(u * math.log(4097.0))).astype(np.int64)
    small = np.clip(small, 1, 4096)
    sizes = np.concatenate([small, np.full(64, 1 << 20, dtype=np.int64)])
    perm = np.random.Generator(np.random.PCG64(seed(5, 0, "perm"))).permutation(sizes.size)
    return [int(x) for x in sizes[perm]]


# ----------------------------------------------------------------------------
# Workload definitions.
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    param_numel: tuple
    bucket_numel: int
    dp_size: int
    verify_ranks: tuple
    time_ranks: tuple
    # replica storage: "world" = D whole padded buffers; "local" = D slices of the rank's shard
    grad_mode: str
    grad_sigma: float
    master_sigma: float
    m_sigma: float          # 0.0 means m starts at zero
    v_sigma: float          # v = (N(0, v_sigma))**2; 0.0 means v starts at zero
    scale: float
    steps: int
    probe_fraction: float = 0.0     # share of replica entries replaced by +-65504
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    notes: str = field(default="", compare=False)

    @property
    def hp(self) -> dict:
        return dict(lr=self.lr, beta1=self.beta1, beta2=self.beta2, eps=self.eps,
                    weight_decay=self.weight_decay)

    @property
    def total_numel(self) -> int:
        return int(sum(self.param_numel))


def _mk() -> dict:
    tiny = Workload(1, "tiny", (120, 300, 80, 250, 150, 100), 1000, 4, (0, 1, 2, 3), (1, 2, 3),
                    "world", 1e-2, 0.02, 0.0, 0.0, 0.25, 10,
                    notes="one bucket of 1000, D=4, shard 250; m=v=0, 10 steps")
    gpt2 = Workload(2, "gpt2_small", tuple(gpt2_small_params()), 40_000_000, 8, tuple(range(8)), (1,),
                    "world", 1e-3, 0.02, 1e-3, 1e-3, 1.0 / 8, 1)
    l8b = Workload(3, "llama3_8b", tuple(llama3_params(4096, 32, 14336, 8, 128256)), 100_000_000, 8,
                   (1,), (1,), "local", 1e-3, 0.02, 1e-3, 1e-3, 1.0 / 8, 1)
    l70b = Workload(4, "llama3_70b", tuple(llama3_params(8192, 80, 28672, 8, 128256)), 200_000_000, 32,
                    (1,), (1,), "local", 1e-3, 0.02, 1e-3, 1e-3, 1.0 / 32, 1)
    frag = Workload(5, "frag", tuple(frag_params()), 4_000_000, 16, tuple(range(16)), tuple(range(16)),
                    "world", 1.0, 0.02, 1.0, 1.0, 0.5, 1, probe_fraction=0.01)
    return {w.name: w for w in (tiny, gpt2, l8b, l70b, frag)}


WORKLOADS = _mk()


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ----------------------------------------------------------------------------
# Generators. All return torch tensors on `device`; bf16 tensors come back as
# torch.bfloat16 (callers view them as int16 / uint16 bit patterns).
# ----------------------------------------------------------------------------

def _gen(seed_value: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_value)
    return g


def normal_f32(n: int, sigma: float, seed_value: int, device="cpu", out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 N(0, sigma**2), drawn in fixed chunks so the stream depends only on (seed, n)."""
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=device)
    g = _gen(seed_value, out.device)
    for s in range(0, n, _GEN_CHUNK):
        e = min(n, s + _GEN_CHUNK)
        torch.randn(e - s, generator=g, device=out.device, dtype=torch.float32, out=out[s:e])
        out[s:e].mul_(sigma)
    return out


def square_normal_f32(n: int, sigma: float, seed_value: int, device="cpu",
                      out: torch.Tensor | None = None) -> torch.Tensor:
    out = normal_f32(n, sigma, seed_value, device, out)
    return out.mul_(out)


def normal_bf16(n: int, sigma: float, seed_value: int, device="cpu", out: torch.Tensor | None = None,
                probe_fraction: float = 0.0, probe_seed: int | None = None) -> torch.Tensor:
    """bf16 N(0, sigma**2): fp32 draws rounded by torch's conversion. With
    probe_fraction > 0, that share of entries (independent Bernoulli draws) is
    replaced by +-65504 with a random sign before the conversion."""
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=device)
    dev = out.device
    g = _gen(seed_value, dev)
    gp = _gen(probe_seed, dev) if probe_fraction > 0 else None
    for s in range(0, n, _GEN_CHUNK):
        e = min(n, s + _GEN_CHUNK)
        x = torch.randn(e - s, generator=g, device=dev, dtype=torch.float32)
        x.mul_(sigma)
        if gp is not None:
            u = torch.rand(e - s, generator=gp, device=dev, dtype=torch.float32)
            sign = torch.rand(e - s, generator=gp, device=dev, dtype=torch.float32)
            probe = torch.where(sign < 0.5, -65504.0, 65504.0)
            x = torch.where(u < probe_fraction, probe, x)
        out[s:e].copy_(x)
        del x
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 bit patterns of a bf16 tensor."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32, copy=False)
