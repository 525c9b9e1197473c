"""Drive a workload through the library: plan a stack, fill its cache through
g4attn_append_kv, and run the per-layer decode or prefill calls of one
layer-stack step.  Used by the benchmark, the smoke check and the GPU tests.

Only the library's kernels touch the data; this module arranges tensors.
"""

from __future__ import annotations

import torch

from . import workloads as W
from .g4attn import Stack


def make_stack(wl: W.Workload, device="cuda") -> Stack:
    return Stack(wl.layers, wl.batch, wl.kv_max, wl.max_chunk, device=device)


def make_paged_stack(wl: W.Workload, page_size: int = 64, spare_pages: int = 8, device="cuda",
                     seed: int = 1234) -> Stack:
    """A paged stack for the workload: every position of every sequence gets a
    page, the pages are a seeded random permutation of a pool with a few spare
    pages, and the pool starts out holding arbitrary bits."""
    kv_max = -(-wl.kv_max // page_size) * page_size
    max_pages = kv_max // page_size
    n_pages = wl.batch * max_pages + spare_pages
    st = Stack(wl.layers, wl.batch, kv_max, wl.max_chunk, device=device, page_size=page_size,
               n_pages=n_pages)
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)[: wl.batch * max_pages]
    st.block_table = perm.to(torch.int32).reshape(wl.batch, max_pages).to(device)
    gd = torch.Generator(device=device).manual_seed(seed)
    st.cache.random_(0, 256, generator=gd)
    return st


def _append_span(stack: Stack, layer: int, rows_k, rows_v, spans, device):
    """Append per-sequence rows [n_kv, n_b, D] at positions spans[b] in chunks
    of at most max_chunk tokens (ragged sequences via n_valid)."""
    B = len(rows_k)
    d = stack.layers[layer]
    chunk = stack.max_chunk
    nmax = max(e - s for s, e in spans)
    if nmax <= 0:
        return
    def pad(rows):
        t = torch.zeros((B, nmax, d.n_kv_heads, d.head_dim), dtype=torch.bfloat16, device=device)
        for b, r in enumerate(rows):
            n = r.shape[1]
            if n:
                t[b, :n] = r.permute(1, 0, 2)
        return t
    pk = pad(rows_k)
    pv = pad(rows_v) if rows_v is not None else None
    for c0 in range(0, nmax, chunk):
        n_new = min(chunk, nmax - c0)
        starts = [s + c0 for s, _ in spans]
        nvalid = [max(0, min(n_new, (e - s) - c0)) for s, e in spans]
        k = pk[:, c0:c0 + n_new].contiguous()
        v = pv[:, c0:c0 + n_new].contiguous() if pv is not None else None
        st = torch.tensor(starts, dtype=torch.int32, device=device)
        nv = torch.tensor(nvalid, dtype=torch.int32, device=device)
        max_end = max(s + n for s, n in zip(starts, nvalid))
        stack.append_kv(layer, k, v, st, nv, max_end_pos=max(max_end, 0))


def fill_cache(stack: Stack, wl: W.Workload, device="cuda", layers=None):
    """Write every owner layer's generated K/V (all positions some query of
    the workload can see, including a prefill chunk's own tokens)."""
    for o in wl.owner_layers():
        if layers is not None and o not in layers:
            continue
        d = wl.layers[o]
        spans = [W.kv_span(wl, o, b) for b in range(wl.batch)]
        ks = [W.kv_rows(wl, o, b, "k", device) for b in range(wl.batch)]
        vs = None if d.k_eq_v else [W.kv_rows(wl, o, b, "v", device) for b in range(wl.batch)]
        _append_span(stack, o, ks, vs, spans, device)
        del ks, vs
    torch.cuda.synchronize(device)


class StepBuffers:
    """Device inputs/outputs of one layer-stack step."""

    def __init__(self, wl: W.Workload, device="cuda"):
        self.wl = wl
        self.q = [W.q_tensor(wl, i, device) for i in range(wl.n_layers)]
        self.out = [torch.empty_like(x) for x in self.q]
        if wl.kind == "decode":
            self.lens = torch.tensor(wl.seq_lens, dtype=torch.int32, device=device)
            self.max_len = max(wl.seq_lens)
        else:
            self.start = torch.tensor(wl.start_pos, dtype=torch.int32, device=device)
            self.max_start = max(wl.start_pos)


def run_step(stack: Stack, bufs: StepBuffers, stream=None, layers=None):
    """One layer-stack step: the per-layer decode (or prefill) calls in order."""
    wl = bufs.wl
    for i in (range(wl.n_layers) if layers is None else layers):
        if wl.kind == "decode":
            stack.decode(i, bufs.q[i], bufs.lens, bufs.max_len, bufs.out[i], stream)
        else:
            stack.prefill(i, bufs.q[i], bufs.start, bufs.max_start, bufs.out[i], stream)
