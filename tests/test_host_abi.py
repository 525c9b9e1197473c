"""Host-side checks of the C-ABI library (CPU only: no kernel is launched).

* every function declared in include/g4attn.h is exported by libg4attn.so;
* owner and key-range resolution through the library's hooks are bit-exact
  with the oracle's independent resolution;
* the cache plan (capacities, slots, shared layers, k_eq_v) has the
  properties the kernels rely on;
* every contract violation the host can see returns its status code before
  any launch.
"""

import math
import os
import re
import subprocess

import numpy as np
import pytest

from decode_attention_gemma_amd import g4attn as G
from decode_attention_gemma_amd import workloads as W
from oracle import attn64 as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "g4attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(G.LIB_PATH),
                                reason="libg4attn.so not built")


def _desc(nq, nkv, d, window=0, keqv=0, owner=-1, scale=None):
    return W.LayerDesc(nq, nkv, d, window, keqv, owner, scale if scale is not None else 1 / math.sqrt(d))


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(g4attn_[a-z_]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 13
    lib = G.load()
    out = subprocess.run(["nm", "-D", "--defined-only", G.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in names:
        assert n in exported, n
        getattr(lib, n)
    # and the binding wraps each of them under the same name
    for n in names:
        assert callable(getattr(G, n)), n


@pytest.fixture
def stack():
    made = []

    def make(layers, max_batch=4, kv_max=256, max_chunk=16):
        h = G.g4attn_stack_create(layers, max_batch, kv_max, max_chunk)
        made.append(h)
        return h
    yield make
    for h in made:
        G.g4attn_stack_destroy(h)


@pytest.mark.parametrize("wl", W.all_workloads(), ids=lambda w: f"cfg{w.cfg_id}-{w.name[:24]}")
def test_owner_resolution_matches_oracle(stack, wl):
    h = stack(wl.layers, wl.batch, wl.kv_max, wl.max_chunk)
    ref = O.resolve_owners(wl.layers)
    assert [G.g4attn_resolve_owner(h, i) for i in range(wl.n_layers)] == ref


def test_owner_resolution_random_stacks(stack):
    rng = np.random.default_rng(3)
    for _ in range(40):
        n = int(rng.integers(2, 12))
        layers = []
        for i in range(n):
            glob = bool(rng.integers(0, 2))
            base = _desc(8, 2, 64, 0 if glob else 16, int(glob))
            owners = [j for j, x in enumerate(layers)
                      if x.kv_owner_layer in (-1, j) and (x.window == 0) == glob]
            if owners and rng.integers(0, 2):
                base = W.LayerDesc(4 * int(rng.integers(1, 3)), 2, 64, base.window, base.k_eq_v,
                                   int(rng.choice(owners)), 0.1)
            layers.append(base)
        h = stack(layers)
        assert [G.g4attn_resolve_owner(h, i) for i in range(n)] == O.resolve_owners(layers)


@pytest.mark.parametrize("window", [0, 1, 7, 8, 64, 1024])
def test_key_range_matches_oracle_bit_exact(stack, window):
    h = stack([_desc(4, 2, 32, window)], kv_max=4096, max_chunk=64)
    for n_keys in (0, 1, 2, 17, 48, 1023, 1024, 1025, 4096):
        for q in sorted({0, 1, n_keys - 1, n_keys, n_keys // 2, n_keys - window, n_keys + 3}):
            if q < 0:
                continue
            assert G.g4attn_key_range(h, 0, q, n_keys) == O.key_range(q, n_keys, window), (q, n_keys)


def _k_offsets(h, layer, b, g, pos, D):
    return [G.g4attn_kv_offset(h, layer, b, g, pos, d)[0] for d in range(D)]


def _v_offsets(h, layer, b, g, pos, D):
    return [G.g4attn_kv_offset(h, layer, b, g, pos, d)[1] for d in range(D)]


def test_capacities_and_offsets(stack):
    layers = [_desc(8, 2, 64, 16), _desc(8, 1, 128, 0, 1), _desc(4, 2, 64, 16, owner=0),
              _desc(8, 1, 128, 0, 1, owner=1), _desc(8, 2, 64, 100)]
    max_batch, kv_max, max_chunk = 3, 500, 24
    h = stack(layers, max_batch, kv_max, max_chunk)
    caps = [G.g4attn_layer_capacity(h, i) for i in range(5)]
    # multiples of 64; sliding: a window plus a chunk fits; global: every position
    assert caps[0] == 64 and caps[1] == 512 and caps[4] == 128
    assert caps[2] == caps[0] and caps[3] == caps[1]
    for i, d in enumerate(layers):
        assert caps[i] % 64 == 0
        if d.window:
            assert caps[i] >= d.window + max_chunk - 1
        else:
            assert caps[i] >= kv_max
    total = G.g4attn_cache_bytes(h)
    # shared layers read exactly their owner's elements; k_eq_v has one plane
    for b in range(max_batch):
        for g in range(2):
            for pos in (0, 5, 63, 64, 200, 499):
                for d in (0, 7, 8, 31, 32, 63):
                    assert G.g4attn_kv_offset(h, 2, b, g, pos, d) == \
                        G.g4attn_kv_offset(h, 0, b, g, pos, d)
        for pos in (0, 300, 499):
            for d in (0, 100, 127):
                ok_, ov = G.g4attn_kv_offset(h, 3, b, 0, pos, d)
                assert (ok_, ov) == G.g4attn_kv_offset(h, 1, b, 0, pos, d) and ok_ == ov
    for layer in (0, 1, 4):
        d = layers[layer]
        D, cap = d.head_dim, caps[layer]
        gk = 1 if d.n_kv_heads > 1 else 0
        seg_k, seg_v = set(), set()
        n_pos = min(cap, kv_max)  # a global plane is rounded up past kv_max
        for pos in range(n_pos):
            ks = _k_offsets(h, layer, 1, gk, pos, D)
            seg_k.update(ks)
            # the ring: position p and p + cap share their storage
            if pos + cap < kv_max:
                assert _k_offsets(h, layer, 1, gk, pos + cap, D) == ks
            if not d.k_eq_v:
                seg_v.update(_v_offsets(h, layer, 1, gk, pos, D))
        # one (sequence, head) segment is a bijection onto cap x D contiguous bf16
        for seg in ([seg_k] + ([seg_v] if not d.k_eq_v else [])):
            assert len(seg) == n_pos * D
            assert all(o % 2 == 0 for o in seg) and max(seg) + 2 <= total
            if n_pos == cap:
                assert max(seg) - min(seg) == 2 * (cap * D - 1)
            else:
                assert max(seg) - min(seg) < 2 * cap * D
        # blocks of 16 slots (K) / 32 slots (V) are contiguous: what one MFMA
        # operand load of the kernels reads
        k0 = min(_k_offsets(h, layer, 1, gk, 16, D))
        blk = {o for p in range(16, 32) for o in _k_offsets(h, layer, 1, gk, p, D)}
        assert blk == set(range(k0, k0 + 2 * 16 * D, 2))
        if not d.k_eq_v:
            v0 = min(_v_offsets(h, layer, 1, gk, 32, D))
            blk = {o for p in range(32, 64) for o in _v_offsets(h, layer, 1, gk, p, D)}
            assert blk == set(range(v0, v0 + 2 * 32 * D, 2))
    # the planes of different owners / kinds never overlap
    spans = []
    for layer in (0, 1, 4):
        d = layers[layer]
        for kind in ((0, 1) if not d.k_eq_v else (0,)):
            offs = [G.g4attn_kv_offset(h, layer, b, g, p, dd)[kind]
                    for b in (0, max_batch - 1) for g in (0, d.n_kv_heads - 1)
                    for p in (0, min(caps[layer], kv_max) - 1) for dd in (0, d.head_dim - 1)]
            spans.append((min(offs), max(offs)))
    spans.sort()
    assert all(a[1] < b[0] for a, b in zip(spans, spans[1:]))


def test_shared_layers_allocate_nothing(stack):
    own = [_desc(8, 2, 64, 32), _desc(8, 1, 128, 0, 1)]
    shared = own + [_desc(8, 2, 64, 32, owner=0), _desc(8, 1, 128, 0, 1, owner=1)] * 3
    a = G.g4attn_cache_bytes(stack(own))
    b = G.g4attn_cache_bytes(stack(shared))
    assert a == b
    c = G.g4attn_cache_bytes(stack(own + [_desc(8, 2, 64, 32)]))
    assert c > a


def test_cache_size_of_12b_decode_stack(stack):
    wl = W.g12b_decode()
    h = stack(wl.layers, wl.batch, wl.kv_max, wl.max_chunk)
    # 40 sliding owners x K+V ring of 1088 slots; 8 global owners x K only
    expect = 40 * 2 * 16 * 8 * 1088 * 256 * 2 + 8 * 16 * 1 * 4096 * 512 * 2
    assert G.g4attn_cache_bytes(h) == expect


# ---------------------------------------------------------------------------
# status codes (nothing is launched: every call fails before its launch)
# ---------------------------------------------------------------------------

def _rc(fn, *args):
    with pytest.raises(G.G4AttnError) as e:
        fn(*args)
    return e.value.code


@pytest.mark.parametrize("layers,code", [
    ([_desc(6, 4, 64)], G.G4ATTN_ERR_DESC),            # n_q % n_kv != 0
    ([_desc(4, 0, 64)], G.G4ATTN_ERR_DESC),            # no kv heads
    ([_desc(4, 2, 64, window=-1)], G.G4ATTN_ERR_DESC),
    ([W.LayerDesc(4, 2, 64, 0, 2, -1, 1.0)], G.G4ATTN_ERR_DESC),
    ([W.LayerDesc(4, 2, 64, 0, 0, -1, float("nan"))], G.G4ATTN_ERR_DESC),
    ([W.LayerDesc(4, 2, 64, 0, 0, -1, float("inf"))], G.G4ATTN_ERR_DESC),
    ([W.LayerDesc(4, 2, 64, 0, 0, -1, 1.0, -1.0)], G.G4ATTN_ERR_DESC),          # softcap < 0
    ([W.LayerDesc(4, 2, 64, 0, 0, -1, 1.0, float("nan"))], G.G4ATTN_ERR_DESC),
    ([W.LayerDesc(4, 2, 64, 0, 0, -1, 1.0, float("inf"))], G.G4ATTN_ERR_DESC),
    ([W.LayerDesc(4, 2, 64, 0, 0, -1, 1.0, 1e-45)], G.G4ATTN_ERR_DESC),         # scale/c overflows
    ([_desc(4, 2, 48)], G.G4ATTN_ERR_UNSUPPORTED),
    ([_desc(4, 2, 1024)], G.G4ATTN_ERR_UNSUPPORTED),
    ([_desc(4, 2, 64, owner=1), _desc(4, 2, 64)], G.G4ATTN_ERR_OWNER),       # later owner
    ([_desc(4, 2, 64), _desc(4, 2, 64, owner=0), _desc(4, 2, 64, owner=1)], G.G4ATTN_ERR_OWNER),
    ([_desc(4, 2, 64), _desc(4, 4, 64, owner=0)], G.G4ATTN_ERR_OWNER),       # n_kv differs
    ([_desc(4, 2, 64), _desc(4, 2, 128, owner=0)], G.G4ATTN_ERR_OWNER),      # head_dim differs
    ([_desc(4, 2, 64), _desc(4, 2, 64, keqv=1, owner=0)], G.G4ATTN_ERR_OWNER),
    ([_desc(4, 2, 64, 8), _desc(4, 2, 64, 16, owner=0)], G.G4ATTN_ERR_OWNER),  # window differs
    ([_desc(4, 2, 64), _desc(4, 2, 64, owner=-2)], G.G4ATTN_ERR_OWNER),
])
def test_create_rejects(layers, code):
    assert _rc(G.g4attn_stack_create, layers, 2, 64, 8) == code
    assert G.g4attn_last_error()


def test_softcap_accepted_and_not_part_of_the_owner_match():
    # a reader may cap its scores while its owner does not (the cap, like the
    # scale, is the reader's own); 0 means no cap
    layers = [W.LayerDesc(4, 2, 64, 8, 0, -1, 0.125, 0.0), W.LayerDesc(4, 2, 64, 8, 0, 0, 1.0, 4.0),
              W.LayerDesc(4, 1, 64, 0, 1, -1, 0.125, 30.0)]
    h = G.g4attn_stack_create(layers, 2, 64, 8)
    try:
        assert [G.g4attn_resolve_owner(h, i) for i in range(3)] == [0, 0, 2]
    finally:
        G.g4attn_stack_destroy(h)


@pytest.mark.parametrize("mb,kv,mc", [(0, 64, 8), (2, 0, 8), (2, 64, 0), (-1, 64, 8)])
def test_create_rejects_sizes(mb, kv, mc):
    assert _rc(G.g4attn_stack_create, [_desc(4, 2, 64)], mb, kv, mc) == G.G4ATTN_ERR_DESC


def test_create_null():
    lib = G.load()
    out = G.c_void_p()
    assert lib.g4attn_stack_create(None, 1, 1, 1, 1, G.byref(out)) == G.G4ATTN_ERR_NULL
    assert lib.g4attn_cache_bytes(None, None) == G.G4ATTN_ERR_NULL


def test_compute_calls_reject_before_launch(stack):
    layers = [_desc(4, 2, 64, 8), _desc(4, 2, 64, 8, owner=0), _desc(4, 1, 64, 0, 1)]
    h = stack(layers, max_batch=4, kv_max=128, max_chunk=16)
    P = 4096  # a non-NULL dummy pointer; no call below reaches a launch
    # unbound
    assert _rc(G.g4attn_decode, h, 0, P, P, 2, 10, P) == G.G4ATTN_ERR_UNBOUND
    assert _rc(G.g4attn_prefill, h, 0, P, P, 2, 16, 0, P) == G.G4ATTN_ERR_UNBOUND
    assert _rc(G.g4attn_append_kv, h, 0, P, P, P, None, 2, 16, 16) == G.G4ATTN_ERR_UNBOUND
    # misaligned / NULL bind
    assert _rc(G.g4attn_bind, h, 4096 + 8, 4096) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_bind, h, None, 4096) == G.G4ATTN_ERR_NULL
    # shared layer cannot append
    assert _rc(G.g4attn_append_kv, h, 1, P, P, P, None, 2, 16, 16) == G.G4ATTN_ERR_SHARED_LAYER
    # the fused decode step follows the append rules, then the decode ones
    assert _rc(G.g4attn_decode_append, h, 1, P, P, P, P, 2, 10, P) == G.G4ATTN_ERR_SHARED_LAYER
    assert _rc(G.g4attn_decode_append, h, 0, P, None, P, P, 2, 10, P) == G.G4ATTN_ERR_NULL
    assert _rc(G.g4attn_decode_append, h, 0, P, P, None, P, 2, 10, P) == G.G4ATTN_ERR_NULL
    assert _rc(G.g4attn_decode_append, h, 2, P, P, P, P, 2, 10, P) == G.G4ATTN_ERR_NULL
    assert _rc(G.g4attn_decode_append, h, 0, P, P, P, P, 2, 10, P) == G.G4ATTN_ERR_UNBOUND
    assert _rc(G.g4attn_decode_append, h, 2, P, P, None, P, 2, 10, P) == G.G4ATTN_ERR_UNBOUND
    assert _rc(G.g4attn_decode_append, h, 3, P, P, P, P, 2, 10, P) == G.G4ATTN_ERR_RANGE
    # k_eq_v takes no V; others need one
    assert _rc(G.g4attn_append_kv, h, 2, P, P, P, None, 2, 16, 16) == G.G4ATTN_ERR_NULL
    assert _rc(G.g4attn_append_kv, h, 0, P, None, P, None, 2, 16, 16) == G.G4ATTN_ERR_NULL
    # ranges
    assert _rc(G.g4attn_decode, h, 3, P, P, 2, 10, P) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_decode, h, -1, P, P, 2, 10, P) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_decode, h, 0, P, P, 5, 10, P) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_decode, h, 0, P, P, 0, 10, P) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_decode, h, 0, P, P, 2, 129, P) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_decode, h, 0, P, P, 2, 0, P) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_prefill, h, 0, P, P, 2, 17, 0, P) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_prefill, h, 0, P, P, 2, 16, 113, P) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_prefill, h, 0, P, P, 2, 16, -1, P) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_append_kv, h, 0, P, P, P, None, 2, 17, 17) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_append_kv, h, 0, P, P, P, None, 2, 16, 129) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_append_kv, h, 0, P, P, P, None, 9, 16, 16) == G.G4ATTN_ERR_RANGE
    # NULL device pointers
    assert _rc(G.g4attn_decode, h, 0, None, P, 2, 10, P) == G.G4ATTN_ERR_NULL
    assert _rc(G.g4attn_decode, h, 0, P, None, 2, 10, P) == G.G4ATTN_ERR_NULL
    assert _rc(G.g4attn_decode, h, 0, P, P, 2, 10, None) == G.G4ATTN_ERR_NULL
    assert _rc(G.g4attn_prefill, h, 0, P, None, 2, 16, 0, P) == G.G4ATTN_ERR_NULL
    assert _rc(G.g4attn_append_kv, h, 0, None, P, P, None, 2, 16, 16) == G.G4ATTN_ERR_NULL
    assert _rc(G.g4attn_append_kv, h, 0, P, P, None, None, 2, 16, 16) == G.G4ATTN_ERR_NULL
    # hooks
    assert _rc(G.g4attn_kv_offset, h, 0, 4, 0, 0, 0) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_kv_offset, h, 0, 0, 2, 0, 0) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_kv_offset, h, 0, 0, 0, 128, 0) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_kv_offset, h, 0, 0, 0, 0, 64) == G.G4ATTN_ERR_RANGE
    assert _rc(G.g4attn_resolve_owner, h, 7) == G.G4ATTN_ERR_RANGE
    assert "out of range" in G.g4attn_last_error()


# ---------------------------------------------------------------------------
# paged cache plan (host only)
# ---------------------------------------------------------------------------

def _paged(layers, max_batch=2, page=64, n_pages=10, max_pages=4, max_chunk=16):
    return G.g4attn_stack_create_paged(layers, max_batch, page, n_pages, max_pages, max_chunk)


@pytest.mark.parametrize("page,n_pages,max_pages,code", [
    (0, 4, 4, G.G4ATTN_ERR_DESC), (32, 4, 4, G.G4ATTN_ERR_DESC), (96, 4, 4, G.G4ATTN_ERR_DESC),
    (64, 0, 4, G.G4ATTN_ERR_DESC), (64, 4, 0, G.G4ATTN_ERR_DESC),
    (64, 4, 1100, G.G4ATTN_ERR_UNSUPPORTED),  # a key range would span > 1022 pages
])
def test_paged_create_rejects(page, n_pages, max_pages, code):
    assert _rc(_paged, [_desc(4, 2, 64)], 2, page, n_pages, max_pages) == code


def test_paged_offsets_match_an_unpaged_segment():
    """Within a page the slots of one KV head sit exactly as in an unpaged
    segment of the same capacity; pages are disjoint, equally spaced blocks of
    each plane; shared layers read their owner's pages; k_eq_v has one plane."""
    layers = [_desc(8, 2, 64, 40), _desc(8, 1, 128, 0, 1), _desc(4, 2, 64, 40, owner=0)]
    page, n_pages = 64, 5
    h = _paged(layers, max_batch=3, page=page, n_pages=n_pages, max_pages=4)
    u = G.g4attn_stack_create([_desc(8, 2, 64, 0), _desc(8, 1, 128, 0, 1)], 1, page, 1)
    try:
        assert [G.g4attn_layer_capacity(h, i) for i in range(3)] == [page] * 3
        total = G.g4attn_cache_bytes(h)
        assert total >= n_pages * page * (2 * 64 * 2 * 2 + 1 * 128 * 2)
        for layer, ulayer, D, nkv in ((0, 0, 64, 2), (1, 1, 128, 1)):
            seen_k, seen_v = set(), set()
            base_k = G.g4attn_page_offset(h, layer, 0, 0, 0, 0)[0]
            ubase = G.g4attn_kv_offset(u, ulayer, 0, 0, 0, 0)
            step = nkv * page * D * 2
            for pg in range(n_pages):
                for g in range(nkv):
                    for s in range(0, page, 7):
                        for d in range(0, D, 5):
                            ok_, ov = G.g4attn_page_offset(h, layer, pg, g, s, d)
                            uk, uv = G.g4attn_kv_offset(u, ulayer, 0, 0, s, d)
                            # same in-segment layout as the unpaged segment
                            assert ok_ - base_k == pg * step + g * page * D * 2 + (uk - ubase[0])
                            if layers[layer].k_eq_v:
                                assert ov == ok_
                            else:
                                assert ov - G.g4attn_page_offset(h, layer, 0, 0, 0, 0)[1] == \
                                    pg * step + g * page * D * 2 + (uv - ubase[1])
                            assert 0 <= ok_ < total and 0 <= ov < total
                            assert ok_ not in seen_k
                            seen_k.add(ok_)
                            seen_v.add(ov)
            if not layers[layer].k_eq_v:
                assert not (seen_k & seen_v)
        # the shared layer reads its owner's pages
        for args in ((0, 0, 3, 9), (4, 1, 63, 63)):
            assert G.g4attn_page_offset(h, 2, *args) == G.g4attn_page_offset(h, 0, *args)
    finally:
        G.g4attn_stack_destroy(h)
        G.g4attn_stack_destroy(u)


def test_paged_calls_reject_before_launch():
    layers = [_desc(4, 2, 64, 8), _desc(4, 1, 64, 0, 1)]
    h = _paged(layers, max_batch=2, page=64, n_pages=6, max_pages=2, max_chunk=16)
    u = G.g4attn_stack_create(layers, 2, 128, 16)
    P = 4096
    try:
        # each kind of stack takes only its own entry points
        assert _rc(G.g4attn_decode, h, 0, P, P, 2, 10, P) == G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_prefill, h, 0, P, P, 2, 16, 0, P) == G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_append_kv, h, 0, P, P, P, None, 2, 16, 16) == G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_decode_append, h, 0, P, P, P, P, 2, 10, P) == G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_kv_offset, h, 0, 0, 0, 0, 0) == G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_decode_paged, u, 0, P, P, 2, 10, P, P) == G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_prefill_paged, u, 0, P, P, 2, 16, 0, P, P) == G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_append_kv_paged, u, 0, P, P, P, None, 2, 16, 16, P) == \
            G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_page_offset, u, 0, 0, 0, 0, 0) == G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_decode_append_paged, u, 0, P, P, P, P, 2, 10, P, P) == \
            G.G4ATTN_ERR_UNSUPPORTED
        assert _rc(G.g4attn_decode_append_paged, h, 0, P, P, P, P, 2, 10, None, P) == \
            G.G4ATTN_ERR_NULL
        assert _rc(G.g4attn_decode_append_paged, h, 1, P, P, P, P, 2, 10, P, P) == \
            G.G4ATTN_ERR_NULL  # k_eq_v layer takes no v_new
        assert _rc(G.g4attn_decode_append_paged, h, 0, P, P, P, None, 2, 10, P, P) == \
            G.G4ATTN_ERR_NULL  # a V plane needs v_new
        assert _rc(G.g4attn_decode_append_paged, h, 0, P, P, P, P, 2, 10, P, P) == \
            G.G4ATTN_ERR_UNBOUND
        # NULL block table, then the unpaged checks in their order
        assert _rc(G.g4attn_decode_paged, h, 0, P, P, 2, 10, None, P) == G.G4ATTN_ERR_NULL
        assert _rc(G.g4attn_prefill_paged, h, 0, P, P, 2, 16, 0, None, P) == G.G4ATTN_ERR_NULL
        assert _rc(G.g4attn_append_kv_paged, h, 0, P, P, P, None, 2, 16, 16, None) == \
            G.G4ATTN_ERR_NULL
        assert _rc(G.g4attn_decode_paged, h, 0, P, P, 2, 10, P, P) == G.G4ATTN_ERR_UNBOUND
        assert _rc(G.g4attn_decode_paged, h, 0, P, P, 2, 129, P, P) == G.G4ATTN_ERR_RANGE
        assert _rc(G.g4attn_prefill_paged, h, 0, P, P, 2, 16, 113, P, P) == G.G4ATTN_ERR_RANGE
        assert _rc(G.g4attn_append_kv_paged, h, 1, P, P, P, None, 2, 16, 16, P) == \
            G.G4ATTN_ERR_NULL  # k_eq_v layer takes no V
        # page hook ranges
        assert _rc(G.g4attn_page_offset, h, 0, 6, 0, 0, 0) == G.G4ATTN_ERR_RANGE
        assert _rc(G.g4attn_page_offset, h, 0, 0, 2, 0, 0) == G.G4ATTN_ERR_RANGE
        assert _rc(G.g4attn_page_offset, h, 0, 0, 0, 64, 0) == G.G4ATTN_ERR_RANGE
        assert _rc(G.g4attn_page_offset, h, 0, 0, 0, 0, 64) == G.G4ATTN_ERR_RANGE
    finally:
        G.g4attn_stack_destroy(h)
        G.g4attn_stack_destroy(u)
