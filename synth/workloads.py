"""The synthetic workloads: shapes, value distributions and hyperparameters.

Each workload is one ZeRO rank's optimizer-side step: N replicas' bf16 gradient
chunks for this rank's shard plus the shard's fp32 master / momentum / variance
and its bf16 working copy.  Values are drawn by :mod:`synth`; nothing here does
optimizer arithmetic.

Recipe (sigma is a standard deviation):
  grads   G_r ~ N(0, 1e-3) per replica r, bf16 (upper 16 bits of the fp32 draw)
  master  P   ~ N(0, 0.02)
  moments M = V = 0 ("cold", first step) or M ~ N(0, 1e-4), V = |N(0, 1e-6)| ("warm")
  Adam    lr 1e-3, beta1 0.9, beta2 0.999, eps 1e-8 (the DeepSpeed config example
          in "Почему training 70B модели требует optimizer sharding (ZeRO-3)?", §8,
          uses the same betas and eps)
  zero mask: a Bernoulli(p) set of positions where every replica's grad is +0
          (parameters that took no gradient this step).

Ragged lists live in per-array arenas: tensor t occupies
[offset_t, offset_t + n_t) of every arena, offsets are multiples of 8 elements,
and the gaps between tensors hold drawn values that the step must not touch.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

import synth

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    step: int
    weight_decay: float
    warm: bool
    n_flat: int = 0                      # flat shard length (0 for a ragged list)
    sizes: tuple = field(default=())     # ragged list: per-tensor lengths
    zero_frac: float = 0.0
    seed: int = 0
    g_sigma: float = 1e-3
    p_sigma: float = 0.02
    m_sigma: float = 1e-4
    v_sigma: float = 1e-6

    @property
    def is_list(self) -> bool:
        return len(self.sizes) > 0

    @property
    def n_params(self) -> int:
        return int(sum(self.sizes)) if self.is_list else self.n_flat

    def hp(self) -> dict:
        return dict(HP, weight_decay=self.weight_decay)

    def layout(self, align: int = 8):
        """(offsets, arena_len): tensor t starts at offsets[t] (a multiple of ``align``)."""
        if not self.is_list:
            return np.zeros(1, dtype=np.int64), self.n_flat
        return arena_layout(self.sizes, align)

    def keys(self):
        s = self.seed
        return dict(P=synth.key(s, synth.KIND_P), M=synth.key(s, synth.KIND_M), V=synth.key(s, synth.KIND_V),
                    MASK=synth.key(s, synth.KIND_MASK),
                    G=[synth.key(s, synth.KIND_GRAD, r) for r in range(self.N)])

    def mask_thresh(self) -> int:
        return synth.mask_threshold(self.zero_frac)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def arena_layout(sizes, align: int = 8):
    sizes = np.asarray(sizes, dtype=np.int64)
    padded = (sizes + (align - 1)) // align * align
    offsets = np.zeros(len(sizes), dtype=np.int64)
    if len(sizes) > 1:
        offsets[1:] = np.cumsum(padded)[:-1]
    return offsets, int(padded.sum())


def llama7b_rank_shard_sizes(layers: int = 32, hidden: int = 4096, ffn: int = 11008, dp: int = 8):
    """Per-layer tensors of a Llama-style 7B model, each sharded 1/dp: 4 attention
    projections hidden x hidden, 3 MLP matrices hidden x ffn, 2 norm vectors."""
    per_layer = [hidden * hidden // dp] * 4 + [hidden * ffn // dp] * 3 + [hidden // dp] * 2
    return tuple(per_layer * layers)


def llama70b_rank_shard_sizes(layers: int = 80, hidden: int = 8192, kv: int = 1024, ffn: int = 28672,
                              dp: int = 64):
    """Per-layer tensors of a Llama-style 70B model with grouped-query attention, each sharded 1/dp:
    q and o hidden x hidden, k and v hidden x kv, 3 MLP matrices hidden x ffn, 2 norm vectors."""
    per_layer = [hidden * hidden // dp, hidden * kv // dp, hidden * kv // dp, hidden * hidden // dp] + \
        [hidden * ffn // dp] * 3 + [hidden // dp] * 2
    return tuple(per_layer * layers)


def log_uniform_sizes(count: int, lo: int, hi: int, seed: int = 0):
    """count sizes, floor(exp(U(ln lo, ln hi))) clamped to [lo, hi]; U from a synth stream."""
    u = synth.uniform_f64(synth.key(seed, synth.KIND_SIZES), 0, count)
    a, b = math.log(lo), math.log(hi)
    return tuple(min(hi, max(lo, int(math.floor(math.exp(a + (b - a) * x))))) for x in u)


# The five workloads.
FLAT_1M_N2 = Workload("flat-1M-N2", N=2, step=1, weight_decay=0.0, warm=False, n_flat=1_048_576)
FLAT_124M_N8 = Workload("flat-124M-N8", N=8, step=100, weight_decay=0.0, warm=True, n_flat=124_000_000)
FLAT_70B_DP64_N64 = Workload("flat-70B/64-N64", N=64, step=5000, weight_decay=0.1, warm=True, n_flat=1_093_750_000)


def list_llama7b_dp8_n8() -> Workload:
    return Workload("list-llama7b/8-N8", N=8, step=1000, weight_decay=0.0, warm=True,
                    sizes=llama7b_rank_shard_sizes())


def list_llama70b_dp64_n64() -> Workload:
    """The 70B/64 shard as per-layer tensors (720 tensors, 1.08B parameters), N=64, warm, step 5000, wd 0.1."""
    return Workload("list-llama70b/64-N64", N=64, step=5000, weight_decay=0.1, warm=True,
                    sizes=llama70b_rank_shard_sizes())


def list_ragged_20000_n16(step: int = 1) -> Workload:
    return Workload(f"list-20000-ragged-N16-t{step}", N=16, step=step, weight_decay=0.0, warm=step > 1,
                    sizes=log_uniform_sizes(20_000, 64, 1 << 20), zero_frac=0.001)


# ------------------------------------------------------------ host inputs
def host_inputs(w: Workload, lo: int, hi: int) -> dict:
    """Arena positions [lo, hi): G (N x len, uint16 bf16 bits), P, M, V (float32)."""
    k = w.keys()
    n = hi - lo
    G = np.empty((w.N, n), dtype=np.uint16)
    for r in range(w.N):
        G[r] = synth.normal_bf16(k["G"][r], lo, n, w.g_sigma, k["MASK"], w.mask_thresh())
    P = synth.normal_f32(k["P"], lo, n, w.p_sigma)
    if w.warm:
        M = synth.normal_f32(k["M"], lo, n, w.m_sigma)
        V = synth.normal_f32(k["V"], lo, n, w.v_sigma, absval=True)
    else:
        M = np.zeros(n, dtype=np.float32)
        V = np.zeros(n, dtype=np.float32)
    return dict(G=G, P=P, M=M, V=V)


def host_inputs_at(w: Workload, idx) -> dict:
    """The same draws at arbitrary arena positions ``idx``."""
    k = w.keys()
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    G = np.empty((w.N, idx.size), dtype=np.uint16)
    for r in range(w.N):
        G[r] = synth.normal_bf16_at(k["G"][r], idx, w.g_sigma, k["MASK"], w.mask_thresh())
    P = synth.normal_f32_at(k["P"], idx, w.p_sigma)
    if w.warm:
        M = synth.normal_f32_at(k["M"], idx, w.m_sigma)
        V = synth.normal_f32_at(k["V"], idx, w.v_sigma, absval=True)
    else:
        M = np.zeros(idx.size, dtype=np.float32)
        V = np.zeros(idx.size, dtype=np.float32)
    return dict(G=G, P=P, M=M, V=V)


# ---------------------------------------------------------- device inputs
def device_inputs(w: Workload, device="cuda", b_fill: int = 0x7FBF) -> dict:
    """Allocate and fill the workload's arenas in device memory.

    Returns dict(G=[N bf16 tensors], P, M, V (fp32), B (bf16 working copy,
    pre-filled with ``b_fill`` bits so untouched positions are recognisable),
    offsets, arena_len)."""
    import torch

    offsets, L = w.layout()
    k = w.keys()
    G = []
    for r in range(w.N):
        g = torch.empty(L, dtype=torch.bfloat16, device=device)
        synth.dev_fill_normal_bf16(g, k["G"][r], 0, w.g_sigma, k["MASK"], w.mask_thresh())
        G.append(g)
    P = torch.empty(L, dtype=torch.float32, device=device)
    synth.dev_fill_normal_f32(P, k["P"], 0, w.p_sigma)
    M = torch.empty(L, dtype=torch.float32, device=device)
    V = torch.empty(L, dtype=torch.float32, device=device)
    if w.warm:
        synth.dev_fill_normal_f32(M, k["M"], 0, w.m_sigma)
        synth.dev_fill_normal_f32(V, k["V"], 0, w.v_sigma, absval=True)
    else:
        M.zero_()
        V.zero_()
    B = torch.full((L,), b_fill, dtype=torch.int16, device=device).view(torch.bfloat16) if b_fill < 0x8000 else \
        torch.full((L,), b_fill - 0x10000, dtype=torch.int16, device=device).view(torch.bfloat16)
    return dict(G=G, P=P, M=M, V=V, B=B, offsets=offsets, arena_len=L)
