"""Gemma-4-shaped attention workloads and their seeded synthetic inputs.

The layer geometries follow the pages' model descriptions:

* E4B: 8 query / 2 KV heads, head_dim 256, sliding window 512, cross-layer
  KV-sharing ("Porting Gemma-4 (2B / 4B / 12B) to AWS Inferentia2",
  introduction table and section 2.1);
* 12B: 48 layers; sliding layers have 16 query / 8 KV heads, head_dim 256 and
  a 1024-key window; global layers have a single KV head of head_dim 512 and
  reuse K as V ("Gemma-4 12B on AWS Inferentia2 -- Tensor-Parallel (TP=2),
  device prefill", "Why this is its own port").

Inputs are synthetic: N(0, 1) draws rounded to bf16, from generators seeded per
(workload, layer, tensor kind, sequence).  No weights or datasets are used.
This module only draws numbers and arranges shapes; it computes no attention.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = [
    "LayerDesc",
    "Workload",
    "tiny_stack",
    "e4b_decode",
    "g12b_decode",
    "g12b_prefill",
    "long_decode",
    "kv_span",
    "kv_rows",
    "q_tensor",
    "all_workloads",
]


@dataclass(frozen=True)
class LayerDesc:
    """Per-layer attention geometry (mirrors the C descriptor)."""

    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int  # 0 = global
    k_eq_v: int  # 1: V rows are the cached K rows
    kv_owner_layer: int  # -1 or own index = owns its cache
    scale: float
    softcap: float = 0.0  # attention-logit cap c: s -> c tanh(s / c); 0 = none


@dataclass
class Workload:
    name: str
    cfg_id: int
    layers: list
    batch: int
    kind: str  # "decode" | "prefill"
    kv_max: int
    max_chunk: int = 64
    seq_lens: list | None = None  # decode: keys incl. the current token
    start_pos: list | None = None  # prefill: cached tokens before the chunk
    n_tok: int = 1
    k_scale: float = 1.0
    outlier_p: float = 0.0
    outlier_mult: float = 8.0
    seed_override: int | None = None
    notes: str = ""

    @property
    def seed(self) -> int:
        return self.seed_override if self.seed_override is not None else 1000 + self.cfg_id

    @property
    def n_layers(self) -> int:
        return len(self.layers)

    def owner(self, layer: int) -> int:
        o = self.layers[layer].kv_owner_layer
        return layer if o in (-1, layer) else o

    def owner_layers(self) -> list[int]:
        return [i for i in range(self.n_layers) if self.owner(i) == i]


def _desc(nq, nkv, d, window, keqv, owner=-1) -> LayerDesc:
    return LayerDesc(nq, nkv, d, window, keqv, owner, 1.0 / math.sqrt(d))


def _latest_owner_of_type(layers: list, i: int, is_global: bool) -> int:
    for j in range(i - 1, -1, -1):
        if layers[j].kv_owner_layer in (-1, j) and (layers[j].window == 0) == is_global:
            return j
    raise ValueError(f"no earlier owner of the same type for layer {i}")


def _share_from(layers: list, first_shared: int) -> list:
    """Layers >= first_shared read the most recent earlier owner of their type."""
    out = list(layers)
    for i in range(first_shared, len(out)):
        o = _latest_owner_of_type(out, i, out[i].window == 0)
        out[i] = replace(out[i], kv_owner_layer=o)
    return out


def _g12b_layers() -> list:
    layers = []
    for i in range(48):
        if i % 6 == 5:
            layers.append(_desc(16, 1, 512, 0, 1))
        else:
            layers.append(_desc(16, 8, 256, 1024, 0))
    return layers


def tiny_stack() -> Workload:
    """Two layers: sliding W=8 (4q/2kv, D=32) and global k_eq_v (4q/1kv, D=64)."""
    layers = [_desc(4, 2, 32, 8, 0), _desc(4, 1, 64, 0, 1)]
    return Workload("tiny 2-layer decode stack", 1, layers, batch=2, kind="decode",
                    kv_max=64, seq_lens=[17, 48])


def e4b_decode() -> Workload:
    """12 layers, 5 sliding (W=512) + 1 global; layers 6-11 KV-shared."""
    layers = [_desc(8, 2, 256, 0 if i % 6 == 5 else 512, 0) for i in range(12)]
    layers = _share_from(layers, 6)
    return Workload("E4B-shaped 12-layer decode stack", 2, layers, batch=1, kind="decode",
                    kv_max=512, seq_lens=[511])


def g12b_decode() -> Workload:
    """12B-shaped 48-layer decode stack, B=16, context U{1024..4096}."""
    lens = np.random.default_rng(1003).integers(1024, 4097, 16).tolist()
    return Workload("12B-shaped 48-layer decode stack", 3, _g12b_layers(), batch=16,
                    kind="decode", kv_max=4096, seq_lens=[int(x) for x in lens])


def g12b_prefill(prefix: int) -> Workload:
    """12B-shaped 64-token prefill chunk after ``prefix`` cached tokens, B=4."""
    return Workload(f"12B-shaped 64-token prefill chunk, prefix {prefix}", 4, _g12b_layers(),
                    batch=4, kind="prefill", kv_max=4096, start_pos=[prefix] * 4, n_tok=64,
                    k_scale=0.25)


def long_decode() -> Workload:
    """12B geometry, layers 20-47 KV-shared, B=64, ragged context U{1..32768}."""
    layers = _share_from(_g12b_layers(), 20)
    lens = np.random.default_rng(1005).integers(1, 32769, 64).tolist()
    return Workload("long-context ragged decode stack", 5, layers, batch=64, kind="decode",
                    kv_max=32768, seq_lens=[int(x) for x in lens], outlier_p=0.01,
                    outlier_mult=8.0)


def tp_rank_layers(layers: list, tp: int) -> list:
    """One tensor-parallel rank's share of a layer stack ("Porting Gemma-4 (2B /
    4B / 12B) to AWS Inferentia2", 2.2: KV heads are split across ranks when
    they divide evenly, so each rank keeps whole query-head groups; "Gemma-4
    12B on AWS Inferentia2 -- Tensor-Parallel (TP=2), device prefill", "The
    recipe": a layer with fewer KV heads than ranks keeps its one KV head on
    both ranks and splits only the query heads).  With fewer KV heads than
    ranks in general, each KV head sits on tp / n_kv ranks and a rank holds
    one KV head and the query heads that read it."""
    out = []
    for d in layers:
        if d.n_q_heads % tp:
            raise ValueError(f"{d.n_q_heads} query heads do not split over {tp} ranks")
        if d.n_kv_heads % tp == 0:
            out.append(replace(d, n_q_heads=d.n_q_heads // tp, n_kv_heads=d.n_kv_heads // tp))
        elif tp % d.n_kv_heads == 0:
            out.append(replace(d, n_q_heads=d.n_q_heads // tp, n_kv_heads=1))
        else:
            raise ValueError(f"{d.n_kv_heads} KV heads and {tp} ranks do not divide")
    return out


def g12b_tp2_rank_decode() -> Workload:
    """One rank of the 12B decode stack at TP=2: sliding 8q/4kv, global 8q/1kv
    (the KV head replicated, G=8); same batch and lengths as the 12B stack."""
    wl = g12b_decode()
    return Workload("12B TP=2 rank 48-layer decode stack", 6, tp_rank_layers(wl.layers, 2),
                    batch=16, kind="decode", kv_max=4096, seq_lens=list(wl.seq_lens))


def e4b_tp2_rank_decode() -> Workload:
    """One rank of the E4B decode stack at TP=2: 4q/1kv, sharing as in E4B."""
    return Workload("E4B TP=2 rank 12-layer decode stack", 7,
                    tp_rank_layers(e4b_decode().layers, 2), batch=1, kind="decode",
                    kv_max=512, seq_lens=[511])


def all_workloads() -> list:
    return [tiny_stack(), e4b_decode(), g12b_decode(), g12b_prefill(0), g12b_prefill(960),
            g12b_prefill(4032), long_decode(), g12b_tp2_rank_decode(), e4b_tp2_rank_decode()]


# ----------------------------------------------------------------------------
# seeded generators
# ----------------------------------------------------------------------------

_KIND = {"q": 1, "k": 2, "v": 3}


def _generator(seed: int, layer: int, kind: str, b: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + layer * 10_007 + _KIND[kind] * 101 + b * 7 + 12345)
                  % (2**62))
    return g


def kv_span(wl: Workload, layer: int, b: int) -> tuple[int, int]:
    """Positions [pos0, end) of sequence b whose K/V the workload defines.

    These are the positions some query of the workload can see (everything
    older than the window is never read, so it is never generated).
    """
    d = wl.layers[layer]
    if wl.kind == "decode":
        L = int(wl.seq_lens[b])
        pos0 = max(0, L - d.window) if d.window > 0 else 0
        return pos0, L
    s = int(wl.start_pos[b])
    pos0 = max(0, s - d.window + 1) if d.window > 0 else 0
    return pos0, s + wl.n_tok


def kv_rows(wl: Workload, layer: int, b: int, kind: str, device="cpu") -> torch.Tensor:
    """bf16 [n_kv, n, D] K (kind='k') or V (kind='v') rows of an owner layer
    for sequence b, positions kv_span(wl, layer, b)."""
    d = wl.layers[layer]
    pos0, end = kv_span(wl, layer, b)
    n = max(end - pos0, 0)
    g = _generator(wl.seed, layer, kind, b, device)
    x = torch.randn((d.n_kv_heads, n, d.head_dim), generator=g, device=device,
                    dtype=torch.float32)
    if wl.outlier_p > 0:
        hit = torch.rand(x.shape, generator=g, device=device) < wl.outlier_p
        x = torch.where(hit, x * wl.outlier_mult, x)
    if kind == "k" and wl.k_scale != 1.0:
        x = x * wl.k_scale
    return x.to(torch.bfloat16)


def q_tensor(wl: Workload, layer: int, device="cpu") -> torch.Tensor:
    """bf16 queries: decode [B, n_q, D]; prefill [B, T, n_q, D]."""
    d = wl.layers[layer]
    g = _generator(wl.seed, layer, "q", 0, device)
    if wl.kind == "decode":
        shape = (wl.batch, d.n_q_heads, d.head_dim)
    else:
        shape = (wl.batch, wl.n_tok, d.n_q_heads, d.head_dim)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
