"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerance for floating point (bf16 output of fp32-accumulated attention on
bf16-rounded inputs), per layer:
  * max |gpu - oracle| <= 1e-2 over every output whose oracle value is below 2
    in magnitude (there half a bf16 unit in the last place is at most 2^-8, so
    the bar is the plain one);
  * over all outputs, max (|gpu - oracle| - u/2) <= 1e-2, where u/2 is half a
    bf16 unit in the last place of the oracle value: the error beyond the
    rounding of the result to the bf16 output type, which no bf16-output kernel
    can avoid (an output of 4.3246 must become 4.3125 or 4.3438, 1.2e-2 away
    or more);
  * ||gpu - oracle||_2 / ||oracle||_2 <= 5e-3.
Index work (owner / key-range resolution, cache offsets) is compared
bit-exactly; a single visible key must return its value row bit-exactly (its
softmax weight is exactly 1).
"""

import math
import sys

import numpy as np
import pytest
import torch

from decode_attention_gemma_amd import g4attn as G
from decode_attention_gemma_amd import harness as H
from decode_attention_gemma_amd import workloads as W
from oracle import attn64 as O

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
REL_L2 = 5e-3
DEV = "cuda"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.load()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _desc(nq, nkv, d, window=0, keqv=0, owner=-1, scale=None, softcap=0.0):
    return W.LayerDesc(nq, nkv, d, window, keqv, owner,
                       scale if scale is not None else 1 / math.sqrt(d), softcap)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def bf16_half_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(ax > 0, 2.0 ** (e - 8), 2.0 ** -134)


def check_close(got, ref, tag):
    g = f64(got) if isinstance(got, torch.Tensor) else got
    assert np.isfinite(g).all(), f"{tag}: non-finite output"
    d = np.abs(g - ref)
    max_abs = float(d.max()) if d.size else 0.0
    small = np.abs(ref) < 2.0
    max_abs_small = float(d[small].max()) if small.any() else 0.0
    excess = float(np.maximum(d - bf16_half_ulp(ref), 0.0).max()) if d.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(g - ref)) / nref if nref > 0 else float(np.linalg.norm(g - ref))
    assert max_abs_small <= MAX_ABS and excess <= MAX_ABS and rel <= REL_L2, (
        f"{tag}: max_abs {max_abs:.3e} (|oracle| < 2: {max_abs_small:.3e}; beyond output "
        f"rounding {excess:.3e}) rel_l2 {rel:.3e}")
    return max_abs, rel


# ---------------------------------------------------------------------------
# oracle evaluation of a workload's outputs on the CPU (inputs regenerated
# from the same seeds; nothing comes from the GPU path except the outputs)
# ---------------------------------------------------------------------------

def oracle_decode(wl, layer, b, q_cpu):
    d = wl.layers[layer]
    o = wl.owner(layer)
    pos0, _ = W.kv_span(wl, o, b)
    K = f64(W.kv_rows(wl, o, b, "k", DEV))
    V = None if d.k_eq_v else f64(W.kv_rows(wl, o, b, "v", DEV))
    return O.decode_sequence(d, q_cpu[b], K, V, wl.seq_lens[b], k_pos0=pos0)


def oracle_prefill(wl, layer, b, q_cpu, tokens=None):
    d = wl.layers[layer]
    o = wl.owner(layer)
    pos0, _ = W.kv_span(wl, o, b)
    K = f64(W.kv_rows(wl, o, b, "k", DEV))
    V = None if d.k_eq_v else f64(W.kv_rows(wl, o, b, "v", DEV))
    start = wl.start_pos[b]
    if tokens is None:
        return O.prefill_sequence(d, q_cpu[b], K, V, start, k_pos0=pos0)
    out = []
    for t in tokens:  # token t of the chunk == decode at start + t + 1 keys
        out.append(O.decode_sequence(d, q_cpu[b, t], K, V, start + t + 1, k_pos0=pos0))
    return np.stack(out)


def run_workload(wl):
    say(f"[gpu] workload cfg{wl.cfg_id}: {wl.name}, B={wl.batch}, layers={wl.n_layers}")
    st = H.make_stack(wl, DEV)
    H.fill_cache(st, wl, DEV)
    bufs = H.StepBuffers(wl, DEV)
    H.run_step(st, bufs)
    torch.cuda.synchronize()
    return st, bufs


# ---------------------------------------------------------------------------
# the benchmark workloads
# ---------------------------------------------------------------------------

def test_tiny_stack_all_outputs():
    wl = W.tiny_stack()
    st, bufs = run_workload(wl)
    for layer in range(wl.n_layers):
        q = f64(bufs.q[layer])
        ref = np.stack([oracle_decode(wl, layer, b, q) for b in range(wl.batch)])
        check_close(bufs.out[layer], ref, f"tiny layer {layer}")
        # the owner / key-range hooks agree with the oracle bit-exactly
        assert G.g4attn_resolve_owner(st.handle, layer) == O.resolve_owners(wl.layers)[layer]
        for L in wl.seq_lens:
            assert G.g4attn_key_range(st.handle, layer, L - 1, L) == \
                O.key_range(L - 1, L, wl.layers[layer].window)


def test_e4b_shared_stack_all_outputs():
    wl = W.e4b_decode()
    st, bufs = run_workload(wl)
    for layer in range(wl.n_layers):
        q = f64(bufs.q[layer])
        ref = np.stack([oracle_decode(wl, layer, b, q) for b in range(wl.batch)])
        check_close(bufs.out[layer], ref, f"e4b layer {layer}")


def test_12b_decode_stack_sampled_layers_all_sequences():
    wl = W.g12b_decode()
    st, bufs = run_workload(wl)
    for layer in (0, 4, 5, 6, 11, 40, 46, 47):
        q = f64(bufs.q[layer])
        ref = np.stack([oracle_decode(wl, layer, b, q) for b in range(wl.batch)])
        m, r = check_close(bufs.out[layer], ref, f"12b decode layer {layer}")
        say(f"  layer {layer}: max_abs {m:.2e} rel {r:.2e}")


@pytest.mark.parametrize("prefix", [0, 960, 4032])
def test_12b_prefill_chunk_sampled(prefix):
    wl = W.g12b_prefill(prefix)
    st, bufs = run_workload(wl)
    for layer in (0, 5, 46, 47):
        q = f64(bufs.q[layer])
        d = wl.layers[layer]
        toks = list(range(64)) if (d.window > 0 or prefix == 0) else [0, 1, 2, 17, 31, 32, 62, 63]
        got = f64(bufs.out[layer])[:, toks]
        ref = np.stack([oracle_prefill(wl, layer, b, q, toks) for b in range(wl.batch)])
        m, r = check_close(got, ref, f"12b prefill P={prefix} layer {layer}")
        say(f"  layer {layer}: max_abs {m:.2e} rel {r:.2e}")


def test_long_context_ragged_sampled():
    wl = W.long_decode()
    st, bufs = run_workload(wl)
    lens = np.array(wl.seq_lens)
    order = np.argsort(lens)
    bs = sorted(set([int(order[0]), int(order[1]), int(order[-1]), int(order[len(order) // 2]),
                     3, 17]))
    for layer in (0, 5, 19, 20, 23, 47):
        q = f64(bufs.q[layer])
        got = f64(bufs.out[layer])[bs]
        ref = np.stack([oracle_decode(wl, layer, b, q) for b in bs])
        m, r = check_close(got, ref, f"long layer {layer}")
        say(f"  layer {layer} (seqs {bs}, lens {lens[bs].tolist()}): max_abs {m:.2e} rel {r:.2e}")


def test_tp2_rank_stacks_sampled():
    """One tensor-parallel rank of the 12B (sliding 8q/4kv, global 8q/1kv
    replicated, G=8) and of the E4B (4q/1kv, KV-shared) stacks."""
    wl = W.g12b_tp2_rank_decode()
    st, bufs = run_workload(wl)
    for layer in (0, 5, 47):
        q = f64(bufs.q[layer])
        ref = np.stack([oracle_decode(wl, layer, b, q) for b in range(wl.batch)])
        m, r = check_close(bufs.out[layer], ref, f"12b rank layer {layer}")
        say(f"  layer {layer}: max_abs {m:.2e} rel {r:.2e}")
    wl = W.e4b_tp2_rank_decode()
    st, bufs = run_workload(wl)
    for layer in range(wl.n_layers):
        q = f64(bufs.q[layer])
        ref = np.stack([oracle_decode(wl, layer, b, q) for b in range(wl.batch)])
        check_close(bufs.out[layer], ref, f"e4b rank layer {layer}")


# ---------------------------------------------------------------------------
# grids of shapes: several tiles, ragged tails, every descriptor branch
# ---------------------------------------------------------------------------

def _custom(layers, batch, kind, kv_max, max_chunk=64, seq_lens=None, start_pos=None, n_tok=1,
            seed=77):
    return W.Workload("custom", 9, layers, batch, kind, kv_max, max_chunk, seq_lens, start_pos,
                      n_tok, seed_override=seed)


DECODE_GRID = [
    # nq, nkv, D, window, keqv, lens
    (4, 2, 32, 8, 0, [1, 2, 9, 17, 48, 64]),
    (4, 1, 64, 0, 1, [1, 65, 130, 257]),
    (8, 8, 128, 0, 0, [1, 63, 64, 65, 500]),
    (16, 8, 256, 100, 0, [99, 100, 101, 333]),
    (16, 1, 512, 0, 1, [1, 300, 777, 1500]),
    (16, 1, 512, 0, 0, [5, 1000]),
    (32, 1, 64, 0, 0, [3, 200]),     # G = 32: two head blocks
    (12, 4, 64, 16, 1, [1, 40]),      # G = 3
    (16, 2, 256, 0, 1, [1, 2, 700]),  # G = 8
]


@pytest.mark.parametrize("nq,nkv,D,window,keqv,lens", DECODE_GRID)
def test_decode_grid(nq, nkv, D, window, keqv, lens):
    say(f"[gpu] decode grid nq={nq} nkv={nkv} D={D} W={window} k_eq_v={keqv} lens={lens}")
    wl = _custom([_desc(nq, nkv, D, window, keqv)], len(lens), "decode", kv_max=2048,
                 seq_lens=lens)
    st, bufs = run_workload(wl)
    q = f64(bufs.q[0])
    ref = np.stack([oracle_decode(wl, 0, b, q) for b in range(wl.batch)])
    check_close(bufs.out[0], ref, "decode grid")
    # a longer host bound changes the split plan, not the result
    out2 = st.decode(0, bufs.q[0], bufs.lens, 2048)
    torch.cuda.synchronize()
    check_close(out2, ref, "decode grid, kv_max bound")


PREFILL_GRID = [
    # nq, nkv, D, window, keqv, T, starts
    (4, 2, 32, 8, 0, 16, [0, 5, 30]),
    (4, 1, 64, 0, 1, 64, [0, 64, 100]),
    (8, 2, 128, 50, 0, 33, [0, 17]),
    (16, 8, 256, 100, 0, 64, [0, 70, 300]),
    (16, 1, 512, 0, 1, 64, [0, 130]),
    (16, 1, 512, 0, 0, 7, [3]),
    (2, 2, 64, 0, 0, 1, [0, 9]),
    (24, 2, 64, 0, 0, 64, [10]),  # G = 12: row blocks straddle tokens
]


@pytest.mark.parametrize("nq,nkv,D,window,keqv,T,starts", PREFILL_GRID)
def test_prefill_grid(nq, nkv, D, window, keqv, T, starts):
    say(f"[gpu] prefill grid nq={nq} nkv={nkv} D={D} W={window} k_eq_v={keqv} T={T} starts={starts}")
    wl = _custom([_desc(nq, nkv, D, window, keqv)], len(starts), "prefill", kv_max=1024,
                 max_chunk=64, start_pos=starts, n_tok=T)
    st, bufs = run_workload(wl)
    q = f64(bufs.q[0])
    ref = np.stack([oracle_prefill(wl, 0, b, q) for b in range(wl.batch)])
    check_close(bufs.out[0], ref, "prefill grid")


def test_sliding_ring_wraps():
    # a ring of 64 slots for window 8: positions far beyond the ring, ragged
    lens = [1, 8, 64, 65, 200, 1000]
    layers = [_desc(4, 2, 64, 8), _desc(4, 2, 64, 8, owner=0, scale=0.3)]
    wl = _custom(layers, len(lens), "decode", kv_max=1024, max_chunk=16, seq_lens=lens)
    st, bufs = run_workload(wl)
    assert st.capacity(0) == 64
    for layer in (0, 1):
        q = f64(bufs.q[layer])
        ref = np.stack([oracle_decode(wl, layer, b, q) for b in range(wl.batch)])
        check_close(bufs.out[layer], ref, f"ring layer {layer}")


def test_prefill_through_ring():
    starts = [0, 40, 500]
    layers = [_desc(8, 2, 64, 24)]
    wl = _custom(layers, 3, "prefill", kv_max=1024, max_chunk=16, start_pos=starts, n_tok=16)
    st, bufs = run_workload(wl)
    assert st.capacity(0) == 64
    q = f64(bufs.q[0])
    ref = np.stack([oracle_prefill(wl, 0, b, q) for b in range(3)])
    check_close(bufs.out[0], ref, "prefill ring")


# ---------------------------------------------------------------------------
# bit-exact index work and closed forms
# ---------------------------------------------------------------------------

def test_append_layout_readback_bit_exact():
    layers = [_desc(4, 2, 64, 8), _desc(4, 1, 128, 0, 1), _desc(4, 2, 64, 8, owner=0)]
    st = G.Stack(layers, max_batch=3, kv_max=256, max_chunk=16, device=DEV)
    cap = st.capacity(0)
    gen = torch.Generator(device=DEV).manual_seed(5)
    written = {}
    for rnd in range(6):  # rounds of up to 16 positions from 0, 40, 120, ring wrap
        starts = [16 * rnd, 40 + 16 * rnd, 120 + 16 * rnd]
        nvalid = [16, 16 if rnd % 2 else 9, 16]
        for layer in (0, 1):
            d = layers[layer]
            k = torch.randn((3, 16, d.n_kv_heads, d.head_dim), generator=gen, device=DEV).to(torch.bfloat16)
            v = None if d.k_eq_v else torch.randn((3, 16, d.n_kv_heads, d.head_dim), generator=gen,
                                                  device=DEV).to(torch.bfloat16)
            st.append_kv(layer, k, v, torch.tensor(starts, dtype=torch.int32, device=DEV),
                         torch.tensor(nvalid, dtype=torch.int32, device=DEV),
                         max_end_pos=max(s + n for s, n in zip(starts, nvalid)))
            for b in range(3):
                for t in range(nvalid[b]):
                    for g in range(d.n_kv_heads):
                        written[(layer, b, g, starts[b] + t)] = (
                            k[b, t, g].cpu(), None if v is None else v[b, t, g].cpu())
    torch.cuda.synchronize()
    cache = st.cache.cpu().view(torch.int16)
    latest = {}
    for (layer, b, g, pos), kv in written.items():
        c = st.capacity(layer)
        latest[(layer, b, g, pos % c)] = (pos, kv)
    n = 0
    for (layer, b, g, slot), (pos, (k, v)) in latest.items():
        D = layers[layer].head_dim
        offs = [G.g4attn_kv_offset(st.handle, layer, b, g, pos, d) for d in range(D)]
        krow = cache[torch.tensor([o[0] // 2 for o in offs])]
        assert torch.equal(krow, k.view(torch.int16)), (layer, b, g, pos)
        if v is not None:
            vrow = cache[torch.tensor([o[1] // 2 for o in offs])]
            assert torch.equal(vrow, v.view(torch.int16))
        else:
            assert all(o[0] == o[1] for o in offs)
        if layer == 0:  # the shared layer reads exactly the owner's elements
            assert G.g4attn_kv_offset(st.handle, 2, b, g, pos, 5) == offs[5]
        n += 1
    assert n > 100
    st.close()


@pytest.mark.parametrize("D,keqv", [(32, 0), (256, 0), (512, 1), (512, 0)])
def test_single_key_returns_value_bit_exact(D, keqv):
    wl = _custom([_desc(16, 1 if D == 512 else 4, D, 0 if keqv else 8, keqv)], 3, "decode",
                 kv_max=64, seq_lens=[1, 1, 1])
    st, bufs = run_workload(wl)
    d = wl.layers[0]
    G_ = d.n_q_heads // d.n_kv_heads
    for b in range(3):
        kind = "k" if keqv else "v"
        val = W.kv_rows(wl, 0, b, kind, DEV)[:, 0]  # [n_kv, D]
        expect = val.repeat_interleave(G_, dim=0)
        assert torch.equal(bufs.out[0][b], expect), b


def test_zero_length_sequences_give_zeros():
    layers = [_desc(4, 2, 64, 0)]
    st = G.Stack(layers, max_batch=3, kv_max=64, max_chunk=16, device=DEV)
    q = torch.randn((3, 4, 64), device=DEV).to(torch.bfloat16)
    lens = torch.tensor([0, -5, 0], dtype=torch.int32, device=DEV)
    out = st.decode(0, q, lens, 8, out=torch.full_like(q, 7.0))
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    st.close()


# ---------------------------------------------------------------------------
# invariants through the GPU path itself
# ---------------------------------------------------------------------------

def test_gqa_equals_mha_with_repeated_kv_on_gpu():
    lens = [37, 300]
    gqa = _custom([_desc(16, 2, 128, 0)], 2, "decode", kv_max=512, seq_lens=lens, seed=5)
    st, bufs = run_workload(gqa)
    mha_layers = [_desc(16, 16, 128, 0)]
    st2 = G.Stack(mha_layers, 2, 512, 64, device=DEV)
    for b, L in enumerate(lens):
        k = W.kv_rows(gqa, 0, b, "k", DEV).repeat_interleave(8, dim=0)  # [16, L, D]
        v = W.kv_rows(gqa, 0, b, "v", DEV).repeat_interleave(8, dim=0)
        H._append_span(st2, 0, [k if i == b else k[:, :0] for i in range(2)],
                       [v if i == b else v[:, :0] for i in range(2)],
                       [(0, L) if i == b else (0, 0) for i in range(2)], DEV)
    out2 = st2.decode(0, bufs.q[0], bufs.lens, max(lens))
    torch.cuda.synchronize()
    check_close(out2, f64(bufs.out[0]), "gqa vs mha (gpu)")


def test_k_eq_v_equals_passing_k_as_v_on_gpu():
    lens = [90, 260]
    a = _custom([_desc(16, 1, 512, 0, 1)], 2, "decode", kv_max=512, seq_lens=lens, seed=9)
    st, bufs = run_workload(a)
    st2 = G.Stack([_desc(16, 1, 512, 0, 0)], 2, 512, 64, device=DEV)
    ks = [W.kv_rows(a, 0, b, "k", DEV) for b in range(2)]
    H._append_span(st2, 0, ks, ks, [(0, L) for L in lens], DEV)
    out2 = st2.decode(0, bufs.q[0], bufs.lens, max(lens))
    torch.cuda.synchronize()
    check_close(out2, f64(bufs.out[0]), "k_eq_v vs K as V (gpu)")


def test_sliding_equals_global_when_window_covers_context_on_gpu():
    lens = [100, 511]
    a = _custom([_desc(8, 2, 256, 512)], 2, "decode", kv_max=512, seq_lens=lens, seed=11)
    b_ = _custom([_desc(8, 2, 256, 0)], 2, "decode", kv_max=512, seq_lens=lens, seed=11)
    _, ba = run_workload(a)
    _, bb = run_workload(b_)
    check_close(ba.out[0], f64(bb.out[0]), "sliding vs global (gpu)")


def test_shared_layer_equals_owner_cache_attended_directly():
    wl = W.e4b_decode()
    st, bufs = run_workload(wl)
    # layer 7 reads owner 4's cache; a fresh stack whose layer 0 owns a cache
    # holding the same K/V gives the same result
    d = wl.layers[7]
    st2 = G.Stack([_desc(d.n_q_heads, d.n_kv_heads, d.head_dim, d.window, d.k_eq_v,
                         scale=d.scale)], 1, wl.kv_max, 64, device=DEV)
    spans = [W.kv_span(wl, 4, 0)]
    H._append_span(st2, 0, [W.kv_rows(wl, 4, 0, "k", DEV)], [W.kv_rows(wl, 4, 0, "v", DEV)],
                   spans, DEV)
    out2 = st2.decode(0, bufs.q[7], bufs.lens, bufs.max_len)
    torch.cuda.synchronize()
    assert torch.equal(out2, bufs.out[7])


def test_graph_replays_match_eager():
    wl = W.tiny_stack()
    st, bufs = run_workload(wl)
    eager = [o.clone() for o in bufs.out]
    for o in bufs.out:
        o.zero_()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        H.run_step(st, bufs)  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        H.run_step(st, bufs, stream=s.cuda_stream)
    for rep in range(4):
        for o in bufs.out:
            o.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(bufs.out, eager):
            assert torch.equal(a, b), rep
        _ = torch.randn(1000, device=DEV).sum().item()  # unrelated eager work between replays


def _replay_check(fn, outs, tag):
    """Capture fn() in a HIP graph on a side stream and replay it four times,
    with unrelated eager work between replays; every replay must reproduce the
    eager outputs bit for bit."""
    torch.cuda.synchronize()
    fn(None)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fn(s.cuda_stream)  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn(s.cuda_stream)
    for rep in range(4):
        for o in outs:
            o.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"{tag}: output {i} differs on replay {rep}"
        _ = torch.randn(1000, device=DEV).sum().item()


def test_graph_replays_cover_merges_caps_paging_and_prefill():
    """Graph replays of decode layers whose splits merge in the kernel (the
    arrival counters must be back at zero after each call) and in the merge
    kernel, a capped KV-shared layer, the paged fused decode step, and a
    prefill chunk."""
    layers = [_desc(16, 8, 256, 100), _desc(16, 1, 512, 0, 1),
              _desc(16, 8, 256, 100, owner=0, softcap=5.0)]
    lens = [5, 333, 2049]
    wl = _custom(layers, len(lens), "decode", kv_max=4096, seq_lens=lens, seed=31)
    st = H.make_stack(wl, DEV)
    H.fill_cache(st, wl, DEV)
    bufs = H.StepBuffers(wl, DEV)
    _replay_check(lambda sid: H.run_step(st, bufs, stream=sid), bufs.out, "decode")
    for i in range(len(layers)):
        q = f64(bufs.q[i])
        ref = np.stack([oracle_decode(wl, i, b, q) for b in range(wl.batch)])
        check_close(bufs.out[i], ref, f"graph decode layer {i}")
    del st
    # paged fused decode step: each replay writes the same token rows again
    pst = H.make_paged_stack(wl, page_size=128, device=DEV, seed=8)
    H.fill_cache(pst, wl, DEV)
    gen = torch.Generator(device=DEV).manual_seed(9)
    knew = [torch.randn((wl.batch, d.n_kv_heads, d.head_dim), generator=gen, device=DEV)
            .to(torch.bfloat16) for d in layers[:2]]
    vnew = [torch.randn((wl.batch, 8, 256), generator=gen, device=DEV).to(torch.bfloat16), None]

    def fused(sid):
        for i in range(2):
            pst.decode_append(i, bufs.q[i], knew[i], vnew[i], bufs.lens, bufs.max_len,
                              bufs.out[i], sid)
        pst.decode(2, bufs.q[2], bufs.lens, bufs.max_len, bufs.out[2], sid)
    _replay_check(fused, bufs.out, "paged fused decode")
    del pst
    torch.cuda.empty_cache()
    # prefill chunk (sliding, global k_eq_v, capped shared)
    wp = _custom(layers, 2, "prefill", kv_max=4096, start_pos=[0, 700], n_tok=64, seed=32)
    sp = H.make_stack(wp, DEV)
    H.fill_cache(sp, wp, DEV)
    pb = H.StepBuffers(wp, DEV)
    _replay_check(lambda sid: H.run_step(sp, pb, stream=sid), pb.out, "prefill")
    for i in range(len(layers)):
        q = f64(pb.q[i])
        ref = np.stack([oracle_prefill(wp, i, b, q, tokens=range(0, 64, 9)) for b in range(2)])
        check_close(f64(pb.out[i])[:, 0:64:9], ref, f"graph prefill layer {i}")


# ---------------------------------------------------------------------------
# robustness of the masking and of the online softmax
# ---------------------------------------------------------------------------

GARBAGE_LAYERS = [
    # nq, nkv, D, window, keqv
    (4, 2, 32, 8, 0),
    (16, 8, 256, 100, 0),
    (16, 1, 512, 0, 1),
    (12, 4, 64, 16, 1),
    (16, 1, 512, 0, 0),
]


@pytest.mark.parametrize("nq,nkv,D,window,keqv", GARBAGE_LAYERS)
def test_cache_slots_outside_the_visible_range_may_hold_any_bits(nq, nkv, D, window, keqv):
    """Slots of a key block that no query may see (older than the window,
    beyond the current length, never written) are filled with all-ones bytes,
    a NaN pattern in bf16: outputs stay finite and equal to the oracle's, in
    decode and in prefill."""
    say(f"[gpu] garbage cache nq={nq} nkv={nkv} D={D} W={window} k_eq_v={keqv}")
    desc = _desc(nq, nkv, D, window, keqv)
    lens = [1, 7, 33, 150, 301]
    wl = _custom([desc], len(lens), "decode", kv_max=512, seq_lens=lens)
    st = H.make_stack(wl, DEV)
    st.cache.fill_(255)
    H.fill_cache(st, wl, DEV)
    bufs = H.StepBuffers(wl, DEV)
    H.run_step(st, bufs)
    torch.cuda.synchronize()
    q = f64(bufs.q[0])
    ref = np.stack([oracle_decode(wl, 0, b, q) for b in range(wl.batch)])
    check_close(bufs.out[0], ref, "decode over garbage cache")

    starts = [0, 21, 130]
    wp = _custom([desc], len(starts), "prefill", kv_max=512, max_chunk=64, start_pos=starts,
                 n_tok=40)
    st = H.make_stack(wp, DEV)
    st.cache.fill_(255)
    H.fill_cache(st, wp, DEV)
    bufs = H.StepBuffers(wp, DEV)
    H.run_step(st, bufs)
    torch.cuda.synchronize()
    q = f64(bufs.q[0])
    ref = np.stack([oracle_prefill(wp, 0, b, q) for b in range(wp.batch)])
    check_close(bufs.out[0], ref, "prefill over garbage cache")


@pytest.mark.parametrize("D,keqv,window", [(256, 0, 0), (512, 1, 0), (64, 0, 40)])
def test_peaked_softmax_many_running_max_updates(D, keqv, window):
    """A large scale makes scores span thousands of units: the running max
    moves often and by far more than the lazy-rescale margin, and the softmax
    is close to one-hot.  Decode and prefill stay within tolerance."""
    say(f"[gpu] peaked softmax D={D} k_eq_v={keqv} W={window}")
    desc = _desc(16, 4 if not keqv else 1, D, window, keqv, scale=3.0)
    lens = [2, 90, 513, 1200]
    wl = _custom([desc], len(lens), "decode", kv_max=2048, seq_lens=lens, seed=5)
    st, bufs = run_workload(wl)
    q = f64(bufs.q[0])
    ref = np.stack([oracle_decode(wl, 0, b, q) for b in range(wl.batch)])
    check_close(bufs.out[0], ref, "peaked decode")
    wp = _custom([desc], 2, "prefill", kv_max=2048, start_pos=[0, 700], n_tok=64, seed=6)
    st, bufs = run_workload(wp)
    q = f64(bufs.q[0])
    ref = np.stack([oracle_prefill(wp, 0, b, q) for b in range(wp.batch)])
    check_close(bufs.out[0], ref, "peaked prefill")


# ---------------------------------------------------------------------------
# attention-logit cap: s -> c tanh(s / c)
# ---------------------------------------------------------------------------

SOFTCAP_GRID = [
    # nq, nkv, D, window, keqv, cap, scale: the cap binds hard (scores of
    # tens of units against c = 30 or 0.5), moderately, or not at all (1e4)
    (16, 8, 256, 100, 0, 30.0, 3.0),
    (16, 1, 512, 0, 1, 5.0, None),
    (16, 1, 512, 0, 0, 30.0, 0.2),
    (8, 2, 64, 0, 0, 0.5, 1.0),
    (4, 2, 32, 8, 0, 1e4, None),
    (12, 4, 64, 16, 1, 2.0, 0.5),
]


@pytest.mark.parametrize("nq,nkv,D,window,keqv,cap,scale", SOFTCAP_GRID)
def test_softcap_decode_and_prefill(nq, nkv, D, window, keqv, cap, scale):
    say(f"[gpu] softcap c={cap} scale={scale} nq={nq} nkv={nkv} D={D} W={window} k_eq_v={keqv}")
    desc = _desc(nq, nkv, D, window, keqv, scale=scale, softcap=cap)
    lens = [1, 17, 100, 333, 1029]
    wl = _custom([desc], len(lens), "decode", kv_max=2048, seq_lens=lens, seed=11)
    st, bufs = run_workload(wl)
    q = f64(bufs.q[0])
    ref = np.stack([oracle_decode(wl, 0, b, q) for b in range(wl.batch)])
    check_close(bufs.out[0], ref, "softcap decode")
    wp = _custom([desc], 3, "prefill", kv_max=2048, start_pos=[0, 37, 900], n_tok=64, seed=12)
    st, bufs = run_workload(wp)
    q = f64(bufs.q[0])
    ref = np.stack([oracle_prefill(wp, 0, b, q) for b in range(wp.batch)])
    check_close(bufs.out[0], ref, "softcap prefill")


def test_softcap_is_the_readers_own_on_shared_and_paged_layers():
    """A shared layer applies its own cap to the owner's cache (the owner has
    none), through the unpaged and the paged cache."""
    layers = [_desc(8, 2, 128, window=60), _desc(8, 2, 128, window=60, owner=0, scale=1.5,
                                                   softcap=4.0)]
    lens = [1, 59, 60, 61, 190]
    wl = W.Workload(cfg_id=91, name="softcap shared", kind="decode", layers=layers,
                    batch=len(lens), kv_max=256, max_chunk=64, seq_lens=lens, start_pos=None,
                    n_tok=1)
    for paged in (False, True):
        st = H.make_paged_stack(wl, page_size=64, device=DEV, seed=3) if paged else \
            H.make_stack(wl, DEV)
        H.fill_cache(st, wl, DEV)
        bufs = H.StepBuffers(wl, DEV)
        H.run_step(st, bufs)
        torch.cuda.synchronize()
        for i in range(2):
            q = f64(bufs.q[i])
            ref = np.stack([oracle_decode(wl, i, b, q) for b in range(wl.batch)])
            check_close(bufs.out[i], ref, f"softcap shared layer {i} paged={paged}")


# ---------------------------------------------------------------------------
# fused decode step: append of the current token + decode in one launch
# ---------------------------------------------------------------------------

FUSED_GRID = [
    # nq, nkv, D, window, keqv, lens, kv_max, max_chunk
    (16, 8, 256, 100, 0, [1, 33, 64, 129, 400], 512, 64),
    (16, 1, 512, 0, 1, [1, 16, 17, 700, 2049], 4096, 64),
    (12, 4, 64, 16, 1, [1, 16, 40, 95], 256, 16),
    (4, 2, 64, 8, 0, [1, 8, 64, 65, 200], 256, 16),   # ring of 64 slots wraps
    (32, 1, 64, 0, 0, [3, 200, 513], 1024, 64),         # two head blocks
    # 16 sequences x 8 KV heads: two 17-block splits per (sequence, KV head),
    # so a wave other than the token block's reader writes the token's rows
    (16, 8, 256, 1024, 0, [1024 + 61 * i for i in range(16)], 2048, 64),
]


@pytest.mark.parametrize("nq,nkv,D,window,keqv,lens,kv_max,max_chunk", FUSED_GRID)
def test_fused_decode_step_equals_append_then_decode(nq, nkv, D, window, keqv, lens, kv_max,
                                                     max_chunk):
    """g4attn_decode_append == g4attn_append_kv of the token + g4attn_decode:
    outputs and the whole cache bit-identical; outputs match the oracle."""
    say(f"[gpu] fused decode nq={nq} nkv={nkv} D={D} W={window} k_eq_v={keqv} lens={lens}")
    desc = _desc(nq, nkv, D, window, keqv)
    wl = _custom([desc], len(lens), "decode", kv_max=kv_max, max_chunk=max_chunk, seq_lens=lens)
    B = wl.batch
    spans = [W.kv_span(wl, 0, b) for b in range(B)]
    ks = [W.kv_rows(wl, 0, b, "k", DEV) for b in range(B)]
    vs = None if keqv else [W.kv_rows(wl, 0, b, "v", DEV) for b in range(B)]
    # the current token (position L - 1) is each sequence's last generated row
    k_new = torch.stack([k[:, -1] for k in ks]).contiguous()
    v_new = None if keqv else torch.stack([v[:, -1] for v in vs]).contiguous()
    older = [(s, e - 1) for s, e in spans]
    stacks = []
    for _ in range(2):
        st = H.make_stack(wl, DEV)
        H._append_span(st, 0, [k[:, :-1] for k in ks],
                       None if keqv else [v[:, :-1] for v in vs], older, DEV)
        stacks.append(st)
    bufs = H.StepBuffers(wl, DEV)
    fused = stacks[0].decode_append(0, bufs.q[0], k_new, v_new, bufs.lens, bufs.max_len)
    pos = (bufs.lens - 1).to(torch.int32)
    stacks[1].append_kv(0, k_new[:, None], None if keqv else v_new[:, None], pos,
                        max_end_pos=bufs.max_len)
    plain = stacks[1].decode(0, bufs.q[0], bufs.lens, bufs.max_len)
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)
    assert torch.equal(stacks[0].cache, stacks[1].cache)
    q = f64(bufs.q[0])
    ref = np.stack([oracle_decode(wl, 0, b, q) for b in range(B)])
    check_close(fused, ref, "fused decode")


@pytest.mark.parametrize("nq,nkv,D,window,keqv,lens,kv_max,max_chunk,page", [
    (16, 8, 256, 100, 0, [1, 33, 64, 129, 400], 512, 64, 64),
    (16, 1, 512, 0, 1, [1, 16, 17, 700, 2049], 4096, 64, 128),
    (12, 4, 64, 16, 1, [1, 16, 40, 95], 256, 16, 64),
    (32, 1, 64, 0, 0, [3, 200, 513], 1024, 64, 192),
    (16, 8, 256, 1024, 0, [1024 + 61 * i for i in range(16)], 2048, 64, 64),
])
def test_paged_fused_decode_step_equals_append_then_decode(nq, nkv, D, window, keqv, lens,
                                                           kv_max, max_chunk, page):
    """g4attn_decode_append_paged == g4attn_append_kv_paged + g4attn_decode_paged
    through the same permuted block table over a pool of arbitrary bits:
    outputs and the whole pool bit-identical; outputs match the oracle."""
    say(f"[gpu] paged fused decode nq={nq} nkv={nkv} D={D} W={window} k_eq_v={keqv} "
        f"lens={lens} page={page}")
    desc = _desc(nq, nkv, D, window, keqv)
    wl = _custom([desc], len(lens), "decode", kv_max=kv_max, max_chunk=max_chunk, seq_lens=lens)
    B = wl.batch
    spans = [W.kv_span(wl, 0, b) for b in range(B)]
    ks = [W.kv_rows(wl, 0, b, "k", DEV) for b in range(B)]
    vs = None if keqv else [W.kv_rows(wl, 0, b, "v", DEV) for b in range(B)]
    k_new = torch.stack([k[:, -1] for k in ks]).contiguous()
    v_new = None if keqv else torch.stack([v[:, -1] for v in vs]).contiguous()
    older = [(s, e - 1) for s, e in spans]
    stacks = []
    for _ in range(2):  # same seed: same block table and the same pool bits
        st = H.make_paged_stack(wl, page_size=page, device=DEV, seed=21)
        H._append_span(st, 0, [k[:, :-1] for k in ks],
                       None if keqv else [v[:, :-1] for v in vs], older, DEV)
        stacks.append(st)
    torch.cuda.synchronize()
    assert torch.equal(stacks[0].cache, stacks[1].cache)
    bufs = H.StepBuffers(wl, DEV)
    fused = stacks[0].decode_append(0, bufs.q[0], k_new, v_new, bufs.lens, bufs.max_len)
    pos = (bufs.lens - 1).to(torch.int32)
    stacks[1].append_kv(0, k_new[:, None], None if keqv else v_new[:, None], pos,
                        max_end_pos=bufs.max_len)
    plain = stacks[1].decode(0, bufs.q[0], bufs.lens, bufs.max_len)
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)
    assert torch.equal(stacks[0].cache, stacks[1].cache)
    q = f64(bufs.q[0])
    ref = np.stack([oracle_decode(wl, 0, b, q) for b in range(B)])
    check_close(fused, ref, "paged fused decode")


# ---------------------------------------------------------------------------
# paged cache: the same kernels through a block table
# ---------------------------------------------------------------------------

def _run_paged(wl, page_size):
    say(f"[gpu] paged cfg{wl.cfg_id}: {wl.name}, page {page_size}")
    st = H.make_paged_stack(wl, page_size=page_size, device=DEV)
    H.fill_cache(st, wl, DEV)
    bufs = H.StepBuffers(wl, DEV)
    H.run_step(st, bufs)
    torch.cuda.synchronize()
    return st, bufs


@pytest.mark.parametrize("name,page", [("tiny", 64), ("e4b", 128), ("tiny", 256)])
def test_paged_decode_equals_unpaged_all_layers(name, page):
    """Same logical K/V through a permuted block table over a pool of
    arbitrary bits: every output bit-identical to the unpaged stack."""
    wl = {"tiny": W.tiny_stack, "e4b": W.e4b_decode}[name]()
    _, ref = run_workload(wl)
    _, got = _run_paged(wl, page)
    for i in range(wl.n_layers):
        assert torch.equal(got.out[i], ref.out[i]), f"{name} layer {i}: paged != unpaged"


def test_paged_12b_decode_and_prefill_sampled():
    """12B shapes (sliding windows starting mid-page, global k_eq_v): paged ==
    unpaged bit for bit on sampled layers, and against the oracle."""
    for wl, layers in ((W.g12b_decode(), (0, 5, 6)), (W.g12b_prefill(960), (0, 5))):
        _, ref = run_workload(wl)
        _, got = _run_paged(wl, 64)
        for i in layers:
            assert torch.equal(got.out[i], ref.out[i]), f"{wl.name} layer {i}: paged != unpaged"
        q = f64(got.q[layers[0]])
        b = wl.batch - 1
        if wl.kind == "decode":
            check_close(got.out[layers[0]][b], oracle_decode(wl, layers[0], b, q), "paged 12b decode")
        else:
            check_close(got.out[layers[0]][b, :4], oracle_prefill(wl, layers[0], b, q, tokens=range(4)),
                        "paged 12b prefill")
        del ref, got
        torch.cuda.empty_cache()


def test_paged_ragged_lengths_against_oracle():
    """Ragged lengths across page boundaries (1, a page edge, +-1 around it,
    window starts inside pages), with page ids shared by sliding and global
    layers, compared with the oracle on every sequence."""
    layers = [_desc(4, 2, 64, window=100), _desc(8, 1, 128, keqv=1), _desc(4, 2, 64, window=100, owner=0)]
    lens = [1, 63, 64, 65, 127, 128, 129, 250]
    wl = W.Workload(cfg_id=90, name="paged ragged", kind="decode", layers=layers, batch=len(lens),
                    kv_max=256, max_chunk=64, seq_lens=lens, start_pos=None, n_tok=1)
    st = H.make_paged_stack(wl, page_size=64, device=DEV, seed=7)
    H.fill_cache(st, wl, DEV)
    bufs = H.StepBuffers(wl, DEV)
    H.run_step(st, bufs)
    torch.cuda.synchronize()
    for i in range(len(layers)):
        q = f64(bufs.q[i])
        ref = np.stack([oracle_decode(wl, i, b, q) for b in range(wl.batch)])
        check_close(bufs.out[i], ref, f"paged ragged layer {i}")


def test_paged_block_table_wider_than_a_workgroup():
    """Block-table rows of 320 entries (20480 positions, 64-slot pages), wider
    than the 256 threads that hold one entry each on the narrow-row path: the
    decode copies the page ids through its loop instead.  Bit-identical to the
    unpaged stack, and against the oracle on every sequence."""
    layers = [_desc(4, 2, 64, window=100), _desc(8, 1, 128, keqv=1)]
    lens = [20000, 300, 17001]
    wl = W.Workload(cfg_id=91, name="paged wide table", kind="decode", layers=layers,
                    batch=len(lens), kv_max=20480, max_chunk=64, seq_lens=lens, start_pos=None,
                    n_tok=1)
    _, ref = run_workload(wl)
    pst, got = _run_paged(wl, 64)
    assert pst.block_table.shape[1] == 320
    for i in range(len(layers)):
        assert torch.equal(got.out[i], ref.out[i]), f"wide table layer {i}: paged != unpaged"
        q = f64(got.q[i])
        want = np.stack([oracle_decode(wl, i, b, q) for b in range(wl.batch)])
        check_close(got.out[i], want, f"paged wide table layer {i}")


def test_length_beyond_hint_is_clamped_and_leaves_no_state():
    """seq_lens above the max_seq_len hint: the kernels treat them as the hint,
    so the call covers only the planned splits, every arrival counter returns
    to zero, and the next valid call is exact.  Layers: a sliding layer whose
    splits merge in the kernel and a global k_eq_v layer whose splits go to the
    merge kernel."""
    layers = [_desc(16, 8, 256, 1024), _desc(16, 1, 512, 0, 1)]
    wl = W.Workload("hint violation", 90, layers, batch=4, kind="decode", kv_max=8192,
                    seq_lens=[8000, 3000, 100, 2500])
    st, bufs = run_workload(wl)
    n_ctr = max(wl.batch * d.n_kv_heads * ((d.n_q_heads // d.n_kv_heads + 15) // 16)
                for d in layers)
    for layer in range(wl.n_layers):
        q = f64(bufs.q[layer])
        ref = np.stack([oracle_decode(wl, layer, b, q) for b in range(wl.batch)])
        for hint in (64, 100, 1000):
            bad = torch.empty_like(bufs.q[layer])
            say(f"[gpu] layer {layer}: lengths {wl.seq_lens} under hint {hint}")
            st.decode(layer, bufs.q[layer], bufs.lens, hint, bad)
            torch.cuda.synchronize()
            assert np.isfinite(f64(bad)).all()
            ctr = st.workspace[: 4 * n_ctr].view(torch.int32)
            assert int(ctr.abs().sum()) == 0, f"counters left at {ctr.tolist()}"
            good = torch.full_like(bufs.q[layer], float("nan"))
            st.decode(layer, bufs.q[layer], bufs.lens, bufs.max_len, good)
            torch.cuda.synchronize()
            check_close(good, ref, f"layer {layer} after a hint-{hint} call")
            assert int(st.workspace[: 4 * n_ctr].view(torch.int32).abs().sum()) == 0
