"""Tensor-parallel rank shapes (host only): one rank's share of a layer.

"Porting Gemma-4 (2B / 4B / 12B) to AWS Inferentia2", 2.2: the KV heads are
split across ranks so that every rank keeps whole groups of query heads;
"Gemma-4 12B on AWS Inferentia2 -- Tensor-Parallel (TP=2), device prefill",
"The recipe": the 12B's global layers, with one KV head, keep it on both
ranks and split only the query heads.
"""

import pytest

from decode_attention_gemma_amd import workloads as W
from oracle import attn64 as O


@pytest.mark.parametrize("tp", [1, 2, 4])
@pytest.mark.parametrize("nq,nkv", [(16, 8), (16, 1), (8, 2), (4, 4)])
def test_rank_maps_reassemble_the_full_layer(tp, nq, nkv):
    full = W.LayerDesc(nq, nkv, 64, 0, 0, -1, 0.125)
    ranks = W.tp_rank_layers([full], tp)
    d = ranks[0]
    assert d.n_q_heads * tp == nq
    for r in range(tp):
        for h in range(d.n_q_heads):
            global_h = r * d.n_q_heads + h
            kv_full = O.kv_head_of(global_h, nq, nkv)
            kv_local = O.kv_head_of(h, d.n_q_heads, d.n_kv_heads)
            if nkv % tp == 0:
                # rank r holds KV heads [r * nkv/tp, (r+1) * nkv/tp)
                assert kv_full == r * d.n_kv_heads + kv_local
            else:
                # each KV head sits on tp / nkv ranks; a rank holds the one
                # its query heads read
                assert d.n_kv_heads == 1 and kv_local == 0
                assert kv_full == r // (tp // nkv)


def test_12b_rank_shapes():
    wl = W.g12b_tp2_rank_decode()
    for i, d in enumerate(wl.layers):
        if i % 6 == 5:
            assert (d.n_q_heads, d.n_kv_heads, d.head_dim, d.k_eq_v) == (8, 1, 512, 1)
        else:
            assert (d.n_q_heads, d.n_kv_heads, d.head_dim, d.window) == (8, 4, 256, 1024)
    assert wl.seq_lens == W.g12b_decode().seq_lens


def test_e4b_rank_keeps_sharing():
    full, rank = W.e4b_decode(), W.e4b_tp2_rank_decode()
    assert [d.kv_owner_layer for d in rank.layers] == [d.kv_owner_layer for d in full.layers]
    assert all((d.n_q_heads, d.n_kv_heads) == (4, 1) for d in rank.layers)
    assert O.resolve_owners(rank.layers) == O.resolve_owners(full.layers)


def test_indivisible_shapes_rejected():
    with pytest.raises(ValueError):
        W.tp_rank_layers([W.LayerDesc(6, 2, 64, 0, 0, -1, 0.125)], 4)
    with pytest.raises(ValueError):
        W.tp_rank_layers([W.LayerDesc(12, 3, 64, 0, 0, -1, 0.125)], 2)
