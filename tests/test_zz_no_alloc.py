"""g4attn_decode_noalloc: the decode entry point that allocates nothing and
uses the library's own per-GPU scratch instead of the bound workspace.

CPU part: its host-side rejections happen before any launch.  GPU part
(marked gpu): two calls in a row through the C ABI, the second with a smaller
input, each bit-identical to g4attn_decode on the same inputs (the same
kernels and split plan) and within the oracle tolerance; a third call repeats
the first after the smaller one, so state left in the shared scratch by an
earlier call cannot leak into a later one.
"""

import math

import numpy as np
import pytest
import torch

from decode_attention_gemma_amd import g4attn as G
from decode_attention_gemma_amd import harness as H
from decode_attention_gemma_amd import workloads as W
from oracle import attn64 as O

DEV = "cuda"


def _desc(nq, nkv, d, window=0, keqv=0):
    return W.LayerDesc(nq, nkv, d, window, keqv, -1, 1 / math.sqrt(d))


def _rc(fn, *a):
    try:
        fn(*a)
        return G.G4ATTN_OK
    except G.G4AttnError as e:
        return e.code


def test_noalloc_rejects_before_launch():
    layers = [_desc(16, 8, 256, 1024), _desc(16, 1, 512, 0, 1)]
    h = G.g4attn_stack_create(layers, 64, 32768, 64)
    try:
        P = 4096
        assert _rc(G.g4attn_decode_noalloc, h, 0, P, P, 2, 10, P) == G.G4ATTN_ERR_UNBOUND
        G.g4attn_bind(h, 4096, 4096)
        assert _rc(G.g4attn_decode_noalloc, h, 2, P, P, 2, 10, P) == G.G4ATTN_ERR_RANGE
        assert _rc(G.g4attn_decode_noalloc, h, 0, P, P, 65, 10, P) == G.G4ATTN_ERR_RANGE
        assert _rc(G.g4attn_decode_noalloc, h, 0, P, P, 2, 32769, P) == G.G4ATTN_ERR_RANGE
        assert _rc(G.g4attn_decode_noalloc, h, 0, None, P, 2, 10, P) == G.G4ATTN_ERR_NULL
        # the 12B-shaped global layer at 64 sequences fits (4 splits each)
    finally:
        G.g4attn_stack_destroy(h)
    # 255 sequences x 16 query heads x 2 splits x 514 floats of partials and
    # (m, l), plus the counters: beyond the 16 MiB scratch
    h = G.g4attn_stack_create([_desc(16, 1, 512, 0, 1)], 255, 32768, 64)
    try:
        G.g4attn_bind(h, 4096, 4096)
        assert _rc(G.g4attn_decode_noalloc, h, 0, 4096, 4096, 255, 32768, 4096) == \
            G.G4ATTN_ERR_UNSUPPORTED
        assert "scratch" in G.g4attn_last_error()
    finally:
        G.g4attn_stack_destroy(h)
    hp = G.g4attn_stack_create_paged(layers, 2, 64, 8, 4, 16)
    try:
        assert _rc(G.g4attn_decode_noalloc, hp, 0, 4096, 4096, 2, 10, 4096) == \
            G.G4ATTN_ERR_UNSUPPORTED
    finally:
        G.g4attn_stack_destroy(hp)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _oracle(wl, layer, q):
    d = wl.layers[layer]
    out = []
    for b in range(wl.batch):
        pos0, _ = W.kv_span(wl, layer, b)
        K = _f64(W.kv_rows(wl, layer, b, "k", DEV))
        V = None if d.k_eq_v else _f64(W.kv_rows(wl, layer, b, "v", DEV))
        out.append(O.decode_sequence(d, q[b], K, V, wl.seq_lens[b], k_pos0=pos0))
    return np.stack(out)


def _check_oracle(got, ref, tag):
    d = np.abs(_f64(got) - ref)
    rel = float(np.linalg.norm(_f64(got) - ref) / np.linalg.norm(ref))
    small = np.abs(ref) < 2.0
    assert float(d[small].max()) <= 1e-2 and rel <= 5e-3, f"{tag}: max {d.max()} rel {rel}"


@pytest.mark.gpu
def test_noalloc_decode_equals_decode_twice_smaller_second():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.load()
    # a sliding layer (splits merged in the kernel) and a 12B-style global
    # k_eq_v layer (splits merged by the merge kernel)
    layers = [_desc(16, 8, 256, 1024), _desc(16, 1, 512, 0, 1)]
    big = W.Workload("noalloc big", 95, layers, batch=8, kind="decode", kv_max=4096,
                     seq_lens=[4096, 1, 3000, 1500, 17, 4000, 2222, 1024])
    small = W.Workload("noalloc small", 96, layers, batch=3, kind="decode", kv_max=4096,
                       seq_lens=[900, 33, 700])
    runs = []
    for wl in (big, small, big):
        print(f"[gpu] noalloc: {wl.name}, B={wl.batch}, lens={wl.seq_lens}", flush=True)
        st = H.make_stack(wl, DEV)
        H.fill_cache(st, wl, DEV)
        bufs = H.StepBuffers(wl, DEV)
        stream = torch.cuda.Stream()
        for layer in range(wl.n_layers):
            ref_out = torch.full_like(bufs.q[layer], float("nan"))
            got = torch.full_like(bufs.q[layer], float("nan"))
            torch.cuda.synchronize()  # the fills ran on torch's current stream
            G.g4attn_decode(st.handle, layer, bufs.q[layer], bufs.lens, wl.batch, bufs.max_len,
                            ref_out, stream)
            G.g4attn_decode_noalloc(st.handle, layer, bufs.q[layer], bufs.lens, wl.batch,
                                    bufs.max_len, got, stream)
            stream.synchronize()
            assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16)), \
                f"{wl.name} layer {layer}: noalloc differs from g4attn_decode"
            _check_oracle(got, _oracle(wl, layer, _f64(bufs.q[layer])),
                          f"{wl.name} layer {layer}")
            runs.append(got.cpu())
        st.close()
    # the repeated first input gives the first call's bits again
    assert torch.equal(runs[0].view(torch.int16), runs[4].view(torch.int16))
    assert torch.equal(runs[1].view(torch.int16), runs[5].view(torch.int16))
