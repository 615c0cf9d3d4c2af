"""Seeded synthetic inputs for attention prefill.

This module only draws random tensors and lays them out; it holds none of the
attention arithmetic, so the GPU path and the CPU oracle can both consume
its output without sharing any computation.

Recipe (the same for every workload):
  * values ~ N(0, 1) drawn in float32 from a torch.Generator seeded with the
    workload's seed, in the order q, k, v, sink, then rounded to the input
    dtype (round to nearest even);
  * sinks ~ N(0, 1), rounded through the input dtype and stored as float32,
    so both sides see the same logit;
  * scale = 1 / sqrt(d);
  * the KV cache of sequence b holds past_len[b] + sq[b] valid keys (the
    cached prefix followed by the chunk's own keys); positions beyond that,
    up to the cache capacity, hold NaN when `poison_tail` is set, so that any
    read of an invalid key shows up in the output.

Layouts: q, out [tokens, h_q, d] (sequences packed back to back);
k_cache, v_cache [batch, h_kv, s_cap, d]; sink [h_q].
"""
from dataclasses import dataclass, field, replace
from typing import List, Optional

import torch

_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Case:
    name: str
    h_q: int
    h_kv: int
    d: int
    sq: List[int]                 # chunk length per sequence
    past: List[int]               # cached prefix length per sequence
    window: int                   # <= 0: no window
    dtype: str = "f16"
    sink: bool = True
    seed: int = 0
    s_cap: Optional[int] = None   # cache capacity; default max(past + sq)
    poison_tail: bool = True
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def batch(self) -> int:
        return len(self.sq)

    @property
    def cap(self) -> int:
        need = max([p + s for p, s in zip(self.past, self.sq)] + [1])
        return max(need, self.s_cap or 0)

    @property
    def tokens(self) -> int:
        return sum(self.sq)

    @property
    def cu_seqlens(self) -> List[int]:
        cu = [0]
        for s in self.sq:
            cu.append(cu[-1] + s)
        return cu

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    @property
    def torch_dtype(self):
        return _DTYPES[self.dtype]

    def with_(self, **kw) -> "Case":
        return replace(self, **kw)


def make(case: Case, device="cpu"):
    """Draw the inputs of `case`.  Returns a dict of tensors on `device`
    (q, k_cache, v_cache, sink or None) plus the host-side metadata."""
    dt = case.torch_dtype
    gen = torch.Generator(device=device)
    gen.manual_seed(case.seed)
    B, hq, hkv, d, cap = case.batch, case.h_q, case.h_kv, case.d, case.cap
    q = torch.randn((case.tokens, hq, d), generator=gen, device=device,
                    dtype=torch.float32).to(dt)
    k = torch.randn((B, hkv, cap, d), generator=gen, device=device,
                    dtype=torch.float32).to(dt)
    v = torch.randn((B, hkv, cap, d), generator=gen, device=device,
                    dtype=torch.float32).to(dt)
    sink = None
    if case.sink:
        sink = torch.randn((hq,), generator=gen, device=device,
                           dtype=torch.float32).to(dt).to(torch.float32)
    if case.poison_tail:
        for b in range(B):
            end = case.past[b] + case.sq[b]
            if end < cap:
                k[b, :, end:, :] = float("nan")
                v[b, :, end:, :] = float("nan")
    return {
        "q": q, "k_cache": k, "v_cache": v, "sink": sink,
        "cu_seqlens": case.cu_seqlens, "past_len": list(case.past),
        "window": case.window, "scale": case.scale,
    }


# ---------------------------------------------------------------------------
# Named workloads (gpt-oss attention geometry: 64 q heads, 8 KV heads, d 64,
# sliding window 128 on every other layer; the ragged batch uses the per-rank
# head counts of a 4-way head-sharded gpt-oss-120b: 16 q heads, 2 KV heads).
# ---------------------------------------------------------------------------
def tiny() -> Case:
    return Case("tiny_h4g1_d64_sq128_w32", h_q=4, h_kv=1, d=64, sq=[128], past=[0],
                window=32, seed=1001)


def full_sq4096() -> Case:
    return Case("gptoss20b_full_sq4096", h_q=64, h_kv=8, d=64, sq=[4096], past=[0],
                window=-1, seed=1002)


def swa_chunk(past: int) -> Case:
    return Case(f"gptoss_swa128_chunk512_past{past}", h_q=64, h_kv=8, d=64, sq=[512],
                past=[past], window=128, seed=1003 + past)


CHUNKED16K_LAYERS = 24
CHUNKED16K_CHUNK = 512
CHUNKED16K_TOKENS = 16384


def chunked16k_layer(layer: int) -> Case:
    """One layer of a 16k prefill run as 32 chunks of 512: the whole 16k
    sequence's q and cache (chunk c uses q rows [512c, 512c + 512) at
    past_len 512c).  Odd layers use window 128, even layers full attention."""
    window = 128 if layer % 2 == 1 else -1
    return Case(f"chunked16k_layer{layer}", h_q=64, h_kv=8, d=64,
                sq=[CHUNKED16K_TOKENS], past=[0], window=window, seed=4000 + layer,
                poison_tail=False)


RAGGED_PREFIX = [0, 128, 1024, 4096, 7168, 8192, 8192, 16384]
RAGGED_EXTEND = [1024 * (i + 1) for i in range(8)]


def ragged_bf16() -> Case:
    return Case("ragged8_h16g2_d128_bf16_w128", h_q=16, h_kv=2, d=128, sq=list(RAGGED_EXTEND),
                past=list(RAGGED_PREFIX), window=128, dtype="bf16", seed=1005)
