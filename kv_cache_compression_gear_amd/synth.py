"""Seeded synthetic K/V tensors shaped like a 7B/8B-class attention layer.

Shared by the tests, the benchmark and the smoke check as the one source of
inputs.  It holds no part of the compression arithmetic: it only draws
numbers.

Recipe (the GEAR pages evaluate on LLaMA/Mistral KV caches, which are not
available here; these draws stand in for them):
  K[b,h] = z * c[h]            z ~ N(0,1) [n,d];  c[h] ~ LogNormal(0, 0.5) [d],
                               with `k_outlier_channels` channels of c[h]
                               (chosen by a per-head random permutation)
                               multiplied by `k_outlier_mult`;
  V[b,h] = z * rho[b,h]        rho ~ LogNormal(0, 0.3) [n], broadcast over d;
  then for K and V alike: each entry, independently with probability 0.01,
  is multiplied by u * sign, u ~ U(10, 20), sign = +-1 with equal odds;
  finally rounded to fp16 (round to nearest even).
Draw order from one torch generator: c, outlier channels (per head), z_K,
mask_K, u_K, sign_K, rho, z_V, mask_V, u_V, sign_V -- each as one tensor in
(batch, head, token, dim) order.  The decode tokens of a streaming run are
drawn afterwards from the same generator, one step at a time, with the same
c[h].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


def _spikes(x: torch.Tensor, g: torch.Generator) -> torch.Tensor:
    mask = torch.rand(x.shape, generator=g, device=x.device) < 0.01
    u = 10.0 + 10.0 * torch.rand(x.shape, generator=g, device=x.device)
    sign = torch.where(torch.rand(x.shape, generator=g, device=x.device) < 0.5, -1.0, 1.0)
    return torch.where(mask, x * u * sign, x)


@dataclass
class KVSynth:
    batch: int
    heads: int
    head_dim: int
    k_outlier_channels: int
    k_outlier_mult: float = 8.0
    seed: int = 0
    device: str = "cpu"
    gen: torch.Generator = field(init=False, repr=False)
    chan: torch.Tensor = field(init=False, repr=False)

    def __post_init__(self):
        self.gen = torch.Generator(device=self.device)
        self.gen.manual_seed(self.seed)
        H, d = self.heads, self.head_dim
        c = torch.exp(0.5 * torch.randn((H, d), generator=self.gen, device=self.device))
        for h in range(H):
            ch = torch.randperm(d, generator=self.gen, device=self.device)[: self.k_outlier_channels]
            c[h, ch] *= self.k_outlier_mult
        self.chan = c

    def prompt(self, seq: int):
        """(K, V) fp16, each [batch, heads, seq, head_dim]."""
        B, H, d, g = self.batch, self.heads, self.head_dim, self.gen
        z = torch.randn((B, H, seq, d), generator=g, device=self.device)
        k = _spikes(z * self.chan[None, :, None, :], g).to(torch.float16)
        del z
        rho = torch.exp(0.3 * torch.randn((B, H, seq), generator=g, device=self.device))
        z = torch.randn((B, H, seq, d), generator=g, device=self.device)
        v = _spikes(z * rho[..., None], g).to(torch.float16)
        return k, v

    def step(self):
        """One decode token: (k_new, v_new) fp16, each [batch, heads, head_dim]."""
        k, v = self.prompt(1)
        return k[:, :, 0].contiguous(), v[:, :, 0].contiguous()

    def queries(self, q_heads: int):
        """q ~ N(0,1) fp16 [batch, q_heads, head_dim]."""
        return torch.randn((self.batch, q_heads, self.head_dim), generator=self.gen,
                           device=self.device).to(torch.float16)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int          # KV heads
    seq: int
    head_dim: int
    bits: int
    group: int
    outlier_ppm: int
    rank: int
    power_iters: int
    chunk_tokens: int = 0
    k_outlier_channels: int = 4
    k_outlier_mult: float = 8.0
    q_heads: int = 0            # 0: same as heads (MHA)
    decode_steps: int = 0
    buf_tokens: int = 64
    fill_rank: int = 2

    def kv_synth(self, device: str = "cpu", seed: int = 0) -> KVSynth:
        return KVSynth(self.batch, self.heads, self.head_dim, self.k_outlier_channels,
                       self.k_outlier_mult, seed=seed, device=device)

    @property
    def num_matrices(self) -> int:
        return 2 * self.batch * self.heads

    @property
    def fp16_bytes(self) -> int:
        return 2 * self.batch * self.heads * self.seq * self.head_dim * 2


# The five workloads: tiny; one 7B-shaped layer; aggressive 2-bit; long context
# in 512-token chunks; streaming decode with grouped-query attention.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 256, 64, 4, 64, 20000, 4, 3, k_outlier_channels=2),
    "7b_layer": Workload("7b_layer", 8, 32, 4096, 128, 4, 128, 20000, 4, 3),
    "2bit": Workload("2bit", 16, 32, 2048, 128, 2, 64, 50000, 8, 4, k_outlier_mult=16.0),
    "long_ctx": Workload("long_ctx", 1, 32, 32768, 128, 4, 128, 10000, 4, 3, chunk_tokens=512),
    "stream_gqa": Workload("stream_gqa", 64, 8, 2048, 128, 4, 128, 20000, 4, 3,
                           q_heads=32, decode_steps=256),
}
