"""Seeded synthetic inputs for HGA routed attention.

This module only draws and rounds numbers; it holds none of the method's
arithmetic (no summaries, no routing, no attention).  Both the HIP path (through
``torch`` device tensors) and the CPU oracle (through float64 numpy views) take
the SAME rounded tensors built here.

Workloads (shapes follow the pages' long-context settings: 32K-128K tokens,
C = 64; the pages use needle-in-a-haystack retrieval, which planted needle
chunks stand in for — no benchmark item is reproduced):

* ``tiny_prefill_fp32``   B=1, 4 heads (MHA), d=64, n=1024, C=64, G=16,
                          sink 1, local 1, k=4, g=8, base 1e4; 3 needle chunks per
                          head shared with 8 later queries each.
* ``decode_32k``          B=8, 32/8 heads, d=128, context 32768, sink 1,
                          local 4, k=16, g=32, bf16; 16 needle chunks per KV head.
* ``prefill_32k``         B=1, 32/8 heads, d=128, n=32768, sink 1, local 2,
                          k=32, g=64, base 5e5, bf16; log-normal key norms.
* ``decode_64k``          B=16, 32/8 heads, context 65536, sink 2, local 4,
                          k=32, g=64, bf16; 32 needle chunks per KV head.
* ``offload_decode_128k`` B=4, 64/8 heads, context 131072, sink 2, local 8,
                          k=64, g=128, bf16; 64 needle chunks per KV head; K/V
                          meant for pinned host memory.

All Q and K are drawn directly as post-RoPE vectors: an isotropic Gaussian is
invariant under rotation, so this equals drawing raw vectors and rotating them.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

SEED_BASE = 20260701


@dataclass(frozen=True)
class Spec:
    name: str
    mode: str                 # "prefill" | "decode"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_tokens: int             # prefill: n; decode: context length L (query at L-1)
    chunk_size: int
    group_size: int
    n_sink: int
    n_local: int
    top_k: int
    top_g: int
    rope_base: float
    dtype: str                # "bf16" | "fp32"
    needles: int = 0          # needle chunks per KV head (decode) / per head (prefill)
    needle_range: str = "candidates"   # "candidates" | "all"
    needle_queries: int = 0   # prefill: later queries sharing each needle direction
    key_lognormal: float = 0.0
    hf_threshold: float = 1.0
    seed: int = SEED_BASE
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny_prefill_fp32": Spec("tiny_prefill_fp32", "prefill", 1, 4, 4, 64, 1024, 64, 16, 1, 1,
                              4, 8, 1e4, "fp32", needles=3, needle_queries=8,
                              seed=SEED_BASE + 1),
    "decode_32k": Spec("decode_32k", "decode", 8, 32, 8, 128, 32768, 64, 16, 1, 4, 16, 32,
                       5e5, "bf16", needles=16, needle_range="candidates", seed=SEED_BASE + 2),
    "prefill_32k": Spec("prefill_32k", "prefill", 1, 32, 8, 128, 32768, 64, 16, 1, 2, 32, 64,
                        5e5, "bf16", key_lognormal=0.3, seed=SEED_BASE + 3),
    "decode_64k": Spec("decode_64k", "decode", 16, 32, 8, 128, 65536, 64, 16, 2, 4, 32, 64,
                       5e5, "bf16", needles=32, needle_range="all", seed=SEED_BASE + 4),
    "offload_decode_128k": Spec("offload_decode_128k", "decode", 4, 64, 8, 128, 131072, 64, 16,
                                2, 8, 64, 128, 5e5, "bf16", needles=64, needle_range="all",
                                seed=SEED_BASE + 5),
}


def spec(name: str, **overrides) -> Spec:
    """A named workload, optionally with fields overridden (smaller test variants)."""
    return replace(WORKLOADS[name], **overrides)


# --------------------------------------------------------------------------- #
# rounding helpers (storage form <-> float64)
# --------------------------------------------------------------------------- #
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form -> exact float64 values."""
    if dtype == "bf16":
        return bf16_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def to_torch(arr: np.ndarray, dtype: str, device="cpu", pin: bool = False):
    """Storage form -> torch tensor of the same values (bfloat16 or float32)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    if pin:
        out = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        out.copy_(t)
        return out
    return t.to(device) if device != "cpu" else t


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def _unit(rng, d):
    v = rng.standard_normal(d)
    return v / np.linalg.norm(v)


# --------------------------------------------------------------------------- #
# generation
# --------------------------------------------------------------------------- #
@dataclass
class Workload:
    spec: Spec
    Q: np.ndarray             # storage form [B, Hq, nq, d]
    K: np.ndarray             # storage form [B, Hkv, n, d]
    V: np.ndarray
    seq_len: np.ndarray       # decode: [B] context lengths; prefill: [B] = n
    needle_chunks: dict       # (b, h) -> array of planted chunk ids

    @property
    def nq(self) -> int:
        return self.Q.shape[2]


def make(s: Spec | str, **overrides) -> Workload:
    """Draw the workload deterministically from its seed."""
    if isinstance(s, str):
        s = spec(s, **overrides)
    elif overrides:
        s = replace(s, **overrides)
    rng = np.random.Generator(np.random.PCG64(s.seed))
    B, Hq, Hkv, d, n, C = s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.n_tokens, s.chunk_size
    gq = Hq // Hkv
    nq = n if s.mode == "prefill" else 1
    small = B * Hkv * n * d <= (1 << 24)
    draw = (lambda shape: rng.standard_normal(shape)) if small else \
        (lambda shape: rng.standard_normal(shape, dtype=np.float32))

    Qf = np.asarray(draw((B, Hq, nq, d)), dtype=np.float64)
    needles = {}
    Kst = np.empty((B, Hkv, n, d), dtype=np.uint16 if s.dtype == "bf16" else np.float32)
    Vst = np.empty_like(Kst)
    n_chunks = n // C
    j_last = (n - 1) // C
    for b in range(B):
        Kb = draw((Hkv, n, d))
        Vb = draw((Hkv, n, d))
        if s.key_lognormal > 0.0:
            Kb = Kb * np.exp(s.key_lognormal * rng.standard_normal((Hkv, n, 1))).astype(Kb.dtype)
        if s.needles and s.mode == "decode":
            lo, hi = ((s.n_sink, j_last - s.n_local) if s.needle_range == "candidates"
                      else (0, n_chunks))
            for h in range(Hkv):
                qs = Qf[b, h * gq:(h + 1) * gq, 0].sum(axis=0)
                u = qs / np.linalg.norm(qs)
                cs = rng.choice(np.arange(lo, hi), size=min(s.needles, hi - lo), replace=False)
                for c in cs:
                    Kb[h, c * C:(c + 1) * C] += (2.0 * u).astype(Kb.dtype)
                needles[(b, h)] = np.sort(cs)
        if s.needles and s.mode == "prefill":
            for h in range(Hkv):
                pool = np.arange(1, max(2, min(14, n_chunks - 2)))
                cs = rng.choice(pool, size=min(s.needles, len(pool)), replace=False)
                for c in cs:
                    u = _unit(rng, d)
                    Kb[h, c * C:(c + 1) * C] += (2.0 * u).astype(Kb.dtype)
                    pos = rng.integers((c + 2) * C, n, size=s.needle_queries)
                    for hq in range(h * gq, (h + 1) * gq):
                        Qf[b, hq, pos] += 2.0 * u
                needles[(b, h)] = np.sort(cs)
        Kst[b] = _store(Kb, s.dtype)
        Vst[b] = _store(Vb, s.dtype)
    Qst = _store(Qf, s.dtype)
    seq_len = np.full(B, n, dtype=np.int32)
    return Workload(s, Qst, Kst, Vst, seq_len, needles)


def hga_config_kwargs(s: Spec) -> dict:
    """Method parameters of a spec as plain keyword arguments."""
    return dict(head_dim=s.head_dim, chunk_size=s.chunk_size, group_size=s.group_size,
                n_sink=s.n_sink, n_local=s.n_local, top_k=s.top_k, top_g=s.top_g,
                rope_base=s.rope_base, hf_threshold=s.hf_threshold)
