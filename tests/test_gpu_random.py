"""Seeded random GPU parity sweep: layer geometry, window, k_eq_v, logit cap,
lengths (empty, single key, window and block edges, long) and the paged or
unpaged cache are drawn at random for decode, prefill and the fused decode
step, and every output row is compared with the fp64 oracle to the same
tolerance as the other parity tests.  The seed of each case is in its test
id."""

import math

import numpy as np
import pytest
import torch

from decode_attention_gemma_amd import g4attn as G
from decode_attention_gemma_amd import harness as H
from decode_attention_gemma_amd import workloads as W
from test_gpu_parity import DEV, check_close, f64, oracle_decode, oracle_prefill, say

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.load()


def _draw(seed):
    r = np.random.default_rng(seed)
    D = int(r.choice([32, 64, 128, 256, 512]))
    keqv = int(r.integers(0, 2))
    n_kv = int(r.choice([1, 2, 4]))
    G_ = int(r.choice([1, 2, 3, 4, 8, 16, 20]))
    window = int(r.choice([0, 0, 1, 7, 64, 100, 513]))
    cap = float(r.choice([0.0, 0.0, 2.0, 30.0]))
    scale = float(r.choice([1 / math.sqrt(D), 0.5, 2.0]))
    paged = bool(r.integers(0, 2))
    return r, W.LayerDesc(G_ * n_kv, n_kv, D, window, keqv, -1, scale, cap), paged


def _lens(r, kv_max, window):
    pool = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, kv_max]
    if window > 0:
        pool += [window - 1, window, window + 1, window + 31]
    pool = [x for x in pool if 1 <= x <= kv_max]
    n = int(r.integers(1, 6))
    out = [int(r.choice(pool)) for _ in range(n)] + [int(r.integers(0, kv_max + 1))]
    return out


def _stack(wl, paged, seed):
    if paged:
        return H.make_paged_stack(wl, page_size=64, device=DEV, seed=seed)
    return H.make_stack(wl, DEV)


@pytest.mark.parametrize("seed", list(range(500, 560)))
def test_random_decode_cases(seed):
    r, desc, paged = _draw(seed)
    kv_max = int(r.choice([100, 128, 640, 1000, 2048]))
    lens = _lens(r, kv_max, desc.window)
    say(f"[gpu] random decode seed={seed} {desc} paged={paged} kv_max={kv_max} lens={lens}")
    wl = W.Workload("random decode", 9, [desc], len(lens), "decode", kv_max, 64, lens,
                    seed_override=seed)
    st = _stack(wl, paged, seed)
    H.fill_cache(st, wl, DEV)
    bufs = H.StepBuffers(wl, DEV)
    H.run_step(st, bufs)
    torch.cuda.synchronize()
    q = f64(bufs.q[0])
    ref = np.stack([oracle_decode(wl, 0, b, q) for b in range(wl.batch)])
    check_close(bufs.out[0], ref, f"random decode seed {seed}")


@pytest.mark.parametrize("seed", list(range(2000, 2040)))
def test_random_prefill_cases(seed):
    r, desc, paged = _draw(seed)
    kv_max = int(r.choice([200, 256, 1000, 1024]))
    T = int(r.choice([1, 7, 16, 64]))
    starts = [int(r.integers(0, kv_max - T + 1)) for _ in range(int(r.integers(1, 4)))]
    say(f"[gpu] random prefill seed={seed} {desc} paged={paged} kv_max={kv_max} T={T} "
        f"starts={starts}")
    wl = W.Workload("random prefill", 9, [desc], len(starts), "prefill", kv_max, 64,
                    start_pos=starts, n_tok=T, seed_override=seed)
    st = _stack(wl, paged, seed)
    H.fill_cache(st, wl, DEV)
    bufs = H.StepBuffers(wl, DEV)
    H.run_step(st, bufs)
    torch.cuda.synchronize()
    q = f64(bufs.q[0])
    ref = np.stack([oracle_prefill(wl, 0, b, q) for b in range(wl.batch)])
    check_close(bufs.out[0], ref, f"random prefill seed {seed}")


@pytest.mark.parametrize("seed", list(range(3000, 3030)))
def test_random_fused_decode_cases(seed):
    """The fused decode step (append of the current token + decode, unpaged or
    paged) on random layers: bit-identical to the unfused pair, outputs and
    cache, and within tolerance of the oracle."""
    r, desc, paged = _draw(seed)
    kv_max = int(r.choice([100, 128, 640, 1000, 2048]))
    lens = [max(1, x) for x in _lens(r, kv_max, desc.window)]
    say(f"[gpu] random fused seed={seed} {desc} paged={paged} kv_max={kv_max} lens={lens}")
    wl = W.Workload("random fused", 9, [desc], len(lens), "decode", kv_max, 64, lens,
                    seed_override=seed)
    keqv = desc.k_eq_v
    spans = [W.kv_span(wl, 0, b) for b in range(wl.batch)]
    ks = [W.kv_rows(wl, 0, b, "k", DEV) for b in range(wl.batch)]
    vs = None if keqv else [W.kv_rows(wl, 0, b, "v", DEV) for b in range(wl.batch)]
    k_new = torch.stack([k[:, -1] for k in ks]).contiguous()
    v_new = None if keqv else torch.stack([v[:, -1] for v in vs]).contiguous()
    older = [(s, e - 1) for s, e in spans]
    stacks = []
    for _ in range(2):
        st = _stack(wl, paged, seed)
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
    ref = np.stack([oracle_decode(wl, 0, b, q) for b in range(wl.batch)])
    check_close(fused, ref, f"random fused seed {seed}")
