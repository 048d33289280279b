"""Seeded synthetic workloads for tests and benchmarks.

Only input generation lives here (no step of the method): target and draft
logits shaped like the SSD pages' Llama-3 (V = 128256) and Qwen-3
(V = 151936) evaluations, per-sequence temperatures, and synthetic cache
payloads (the draft transformer that would produce them is out of scope).
Both the GPU path and the CPU oracle consume exactly these tensors.

Recipes (all randomness from torch.Generator(device).manual_seed(1000*cfg + step)):
  1 tiny verify   B=1,   K=4, V=1000,   fp32: z_t ~ N(0, 2^2); z_d = z_t + N(0, 0.5^2)
  2 Llama-3 vocab B=16,  K=5, V=128256, bf16: z_t ~ N(0,1), 8 distinct uniform
                  'peak' tokens per row get +6; z_d = z_t + N(0, 0.8^2)
  3 Qwen-3 vocab  B=64,  K=7, V=151936, bf16: z_t = Gumbel(0,1) - 1.1 ln(rank),
                  rank a uniform random permutation of 1..V per row (Zipf s=1.1
                  offsets); z_d = z_t + N(0, 1)
  4 cache scale   B=256, K=5, V=128256, bf16: as 2; cache budget 64, ratio 0.6
  5 mixed greedy  B=512, K=4, V=151936, fp16: target as 3; z_d = z_t + N(0, 1.5^2);
                  sequences b < 256 greedy (T = 0), b >= 256 at T = 1.2
Noise is added in fp32; the final cast to bf16/fp16 rounds to nearest even.
"""
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Config:
    cfg: int
    name: str
    B: int
    K: int
    V: int
    dtype: torch.dtype
    T: float
    F: int
    C: float
    steps: int
    base_seed: int
    kind: str            # "normal", "peaks", "zipf"
    draft_sd: float
    target_sd: float = 1.0
    F_out: int = 0       # 0 -> F
    Bgt: int = 0         # speculation-cache budget (0: no cache in the workload)
    ratio: float = 0.0
    greedy_half: bool = False

    @property
    def rows(self):
        return self.B * (self.K + 1)

    @property
    def fout(self):
        return self.F_out or self.F


CONFIGS = {
    1: Config(1, "tiny-verify", 1, 4, 1000, torch.float32, 1.0, 2, 0.5, 1000, 0, "normal", 0.5, target_sd=2.0),
    2: Config(2, "llama3-vocab", 16, 5, 128256, torch.bfloat16, 0.7, 4, 0.6, 200, 2, "peaks", 0.8),
    3: Config(3, "qwen3-vocab", 64, 7, 151936, torch.bfloat16, 1.0, 4, 0.5, 100, 3, "zipf", 1.0),
    4: Config(4, "cache-scale", 256, 5, 128256, torch.bfloat16, 0.7, 4, 0.6, 100, 4, "peaks", 0.8,
              F_out=27, Bgt=64, ratio=0.6),
    5: Config(5, "mixed-greedy", 512, 4, 151936, torch.float16, 1.2, 8, 0.3, 100, 5, "zipf", 1.5,
              greedy_half=True),
}


def custom(B, K, V, dtype=torch.bfloat16, T=1.0, F=4, C=0.5, kind="normal", draft_sd=1.0, target_sd=1.0,
           F_out=0, base_seed=7, greedy_half=False, Bgt=0, ratio=0.0):
    """An ad-hoc workload (edge-case and scaling tests)."""
    return Config(0, f"custom-B{B}-K{K}-V{V}", B, K, V, dtype, T, F, C, 1, base_seed, kind, draft_sd,
                  target_sd=target_sd, F_out=F_out, greedy_half=greedy_half, Bgt=Bgt, ratio=ratio)


def _gen(cfg, step, device):
    g = torch.Generator(device=device)
    g.manual_seed(1000 * cfg.cfg + step + 7919 * cfg.base_seed * (cfg.cfg == 0))
    return g


def logits(cfg, step, device):
    """(target, draft) logits [B, K+1, V] in cfg.dtype on `device`."""
    g = _gen(cfg, step, device)
    shape = (cfg.B, cfg.K + 1, cfg.V)
    rows = cfg.rows
    if cfg.kind == "zipf":
        e = torch.empty(shape, device=device).exponential_(generator=g).clamp_min_(1e-30)
        t = -torch.log(e)                                      # Gumbel(0, 1)
        rank = torch.rand((rows, cfg.V), device=device, generator=g).argsort(dim=1).view(shape) + 1
        t -= 1.1 * torch.log(rank.to(torch.float32))
        del rank, e
    else:
        t = torch.randn(shape, device=device, generator=g) * cfg.target_sd
        if cfg.kind == "peaks":
            pk = torch.rand((rows, cfg.V), device=device, generator=g).topk(8, dim=1).indices
            t.view(rows, cfg.V).scatter_add_(1, pk, torch.full(pk.shape, 6.0, device=device))
    d = t + torch.randn(shape, device=device, generator=g) * cfg.draft_sd
    return t.to(cfg.dtype), d.to(cfg.dtype)


def temperatures(cfg, device):
    T = torch.full((cfg.B,), cfg.T, dtype=torch.float32, device=device)
    if cfg.greedy_half:
        T[: cfg.B // 2] = 0.0
    return T


def seed(cfg, step):
    """Philox key of a step: (base_seed << 32) | step."""
    return (cfg.base_seed << 32) | step


def payload(cfg, nslots, step, device):
    """Synthetic pre-speculated tokens [B, nslots, K] (stand-in for the draft's
    per-branch continuations)."""
    g = _gen(cfg, 10 ** 6 + step, device)
    return torch.randint(0, cfg.V, (cfg.B, nslots, cfg.K), generator=g, device=device, dtype=torch.int32)
