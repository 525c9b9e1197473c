"""fp64 CPU reference for Gemma-4-style attention over a KV cache.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the
package-level smoke check and the benchmark's CPU-baseline leg may import or
call this module.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or constant generators) and never imports it.

What it computes is the plain definition of masked softmax attention, one
query head and one query position at a time, in float64:

    out[h] = sum_k w_k * Vhat[k] / sum_k w_k,
    w_k    = exp(s_k - max_k s_k),
    s_k    = scale * <q[h], K[g(h), k]>,         k in the visible key set,
    s_k   <- c * tanh(s_k / c)                     when the layer sets a logit cap c > 0,

with the Gemma-4 specifics described on these pages:

  [FR]  "Porting Gemma-4 (2B / 4B / 12B) to AWS Inferentia2" (dev.to field
        report): the model comparison table in its introduction; section 2.1
        (cross-layer KV-sharing); section 2.2 (GQA under tensor parallelism);
        section 2.3 (the 12B's mixed attention types); section 5 (the
        device-resident KV cache with prefill and decode graphs).
  [FIVE] "Five Gemma-4 models, one accelerator: what porting E2B -> 31B to AWS
        Inferentia2 taught me": "What makes each one different".
  [12B] "Gemma-4 12B on AWS Inferentia2 -- Tensor-Parallel (TP=2), device
        prefill": "Why this is its own port" and "The recipe".

Readings taken where the pages leave a step open (each is repeated at the
function that uses it):
  * window W > 0 means a query at position p sees key positions k with
    p - W < k <= p: W keys counting its own; W == 0 means global causal;
  * in decode, n_keys counts the cached keys including the current token,
    which sits at position n_keys - 1;
  * query head h reads KV head h // (n_q / n_kv) (contiguous groups);
  * attention_k_eq_v: the value rows are the cached key rows themselves;
  * a KV-shared layer reads the cache of an earlier layer that owns its cache
    and has the same (n_kv_heads, head_dim, k_eq_v, window); the mask and the
    scale stay the reader's own;
  * a query that sees no key returns zeros;
  * an attention-logit cap c > 0 (optional; the E4B Inferentia2 model card,
    "Architecture", lists an attention softcap among the recipe's pieces but
    gives no value) bends each scaled score s into c * tanh(s / c) before the
    softmax, the same form the pages give for the final-logit cap; c = 0 or an
    absent field means no cap.

Every function here is pinned by CPU tests against closed forms, invariants,
brute force and a library routine; none is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "OracleError",
    "resolve_owners",
    "key_range",
    "kv_head_of",
    "attend",
    "decode_sequence",
    "prefill_sequence",
]


class OracleError(ValueError):
    """A layer stack that the method does not define."""


def _field(desc, name, default=None):
    if isinstance(desc, dict):
        return desc[name] if default is None else desc.get(name, default)
    return getattr(desc, name) if default is None else getattr(desc, name, default)


def resolve_owners(layers) -> list[int]:
    """Index of the layer whose cache each layer reads.

    [FR] section 2.1: layers flagged as KV-shared run no K/V projection and
    attend to the K/V an earlier layer produced; only the remaining layers hold
    a cache.  [FIVE] "What makes each one different": the E-family layers
    borrow a neighbour's K/V.

    A layer owns its cache when ``kv_owner_layer`` is -1 or its own index.
    Otherwise the named layer must come earlier, must own its cache (no
    chains) and must have the same (n_kv_heads, head_dim, k_eq_v, window).
    """
    owners: list[int] = []
    for i, d in enumerate(layers):
        o = int(_field(d, "kv_owner_layer"))
        if o == -1 or o == i:
            owners.append(i)
            continue
        if o < 0 or o >= i:
            raise OracleError(f"layer {i}: owner {o} is not an earlier layer")
        od = layers[o]
        oo = int(_field(od, "kv_owner_layer"))
        if not (oo == -1 or oo == o):
            raise OracleError(f"layer {i}: owner {o} is itself KV-shared")
        for name in ("n_kv_heads", "head_dim", "k_eq_v", "window"):
            if int(_field(od, name)) != int(_field(d, name)):
                raise OracleError(f"layer {i}: {name} differs from owner {o}")
        owners.append(o)
    return owners


def key_range(q_pos: int, n_keys: int, window: int) -> tuple[int, int]:
    """Half-open range [lo, hi) of key positions a query at ``q_pos`` sees.

    [FR] introduction table and [12B] "Why this is its own port": layers are
    either sliding-window (512 on E2B/E4B, 1024 on the 12B) or global, and
    attention is causal.  Reading: the window counts the query's own key, so a
    query at p sees p - W < k <= p; only the first ``n_keys`` positions exist.
    """
    hi = max(min(q_pos + 1, n_keys), 0)
    lo = max(0, q_pos - window + 1) if window > 0 else 0
    if hi < lo:
        lo = hi
    return lo, hi


def kv_head_of(h: int, n_q: int, n_kv: int) -> int:
    """KV head read by query head ``h``.

    [FR] section 2.2: attention broadcasts each KV head to a group of
    n_q / n_kv query heads; the sharding rule there only keeps the right
    query-to-KV pairing when the groups are contiguous blocks of heads.
    """
    if n_q % n_kv != 0:
        raise OracleError("n_q_heads must be a multiple of n_kv_heads")
    return h // (n_q // n_kv)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           softcap: float = 0.0) -> np.ndarray:
    """Softmax attention of one query vector over the given key/value rows.

    q: [D]; K: [n, D]; V: [n, Dv]; all float64.  n == 0 gives zeros.
    softcap c > 0: each scaled score s becomes c * tanh(s / c) before the
    softmax (the cap form the pages give for Gemma-4's logits, here on the
    attention scores); 0 leaves the scores as they are.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = scale * (K @ q)
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def _rows(X: np.ndarray, k_pos0: int, lo: int, hi: int) -> np.ndarray:
    a, b = lo - k_pos0, hi - k_pos0
    if hi > lo and (a < 0 or b > X.shape[-2]):
        raise OracleError(f"key rows [{lo},{hi}) not provided (have from {k_pos0})")
    return X[..., a:b, :] if hi > lo else X[..., 0:0, :]


def decode_sequence(desc, q: np.ndarray, K: np.ndarray, V, n_keys: int,
                    k_pos0: int = 0) -> np.ndarray:
    """One decode step of one sequence for one layer.

    desc: the reading layer's geometry (n_q_heads, n_kv_heads, head_dim,
          window, k_eq_v, scale, and optionally softcap).
    q:    [n_q, D] query of the current token.
    K, V: [n_kv, n, D] key/value rows of the owning layer's cache for the
          positions k_pos0 .. k_pos0 + n - 1 (V is ignored when k_eq_v).
    n_keys: keys in the cache including the current token, whose position is
          n_keys - 1 ([FR] section 5: the decode graph writes the token's K/V
          into the resident cache and attends to it).
    [12B] "Why this is its own port": with attention_k_eq_v the global layers
    use K in place of V.
    Returns [n_q, D] float64.
    """
    n_q = int(_field(desc, "n_q_heads"))
    n_kv = int(_field(desc, "n_kv_heads"))
    window = int(_field(desc, "window"))
    keqv = int(_field(desc, "k_eq_v"))
    scale = float(_field(desc, "scale"))
    softcap = float(_field(desc, "softcap", 0.0))
    D = int(_field(desc, "head_dim"))
    out = np.zeros((n_q, D), dtype=np.float64)
    if n_keys <= 0:
        return out
    lo, hi = key_range(n_keys - 1, n_keys, window)
    for h in range(n_q):
        g = kv_head_of(h, n_q, n_kv)
        Kh = _rows(K[g], k_pos0, lo, hi)
        Vh = Kh if keqv else _rows(V[g], k_pos0, lo, hi)
        out[h] = attend(q[h], Kh, Vh, scale, softcap)
    return out


def prefill_sequence(desc, q: np.ndarray, K: np.ndarray, V, start: int,
                     k_pos0: int = 0) -> np.ndarray:
    """A chunk of T new tokens of one sequence for one layer.

    q:    [T, n_q, D]: token t sits at position start + t.
    K, V: [n_kv, n, D] rows for positions k_pos0 .. k_pos0 + n - 1 of the
          owning layer, which must already hold the chunk's own keys
          ([FR] section 5 and [12B] "The recipe": one resident cache is filled
          by a prefill bucket of 64 tokens and read by the decode bucket).
    Token t attends causally: keys up to its own position, within the window.
    Returns [T, n_q, D] float64.
    """
    T = q.shape[0]
    n_q = int(_field(desc, "n_q_heads"))
    n_kv = int(_field(desc, "n_kv_heads"))
    window = int(_field(desc, "window"))
    keqv = int(_field(desc, "k_eq_v"))
    scale = float(_field(desc, "scale"))
    softcap = float(_field(desc, "softcap", 0.0))
    D = int(_field(desc, "head_dim"))
    out = np.zeros((T, n_q, D), dtype=np.float64)
    n_keys = start + T
    for t in range(T):
        lo, hi = key_range(start + t, n_keys, window)
        for h in range(n_q):
            g = kv_head_of(h, n_q, n_kv)
            Kh = _rows(K[g], k_pos0, lo, hi)
            Vh = Kh if keqv else _rows(V[g], k_pos0, lo, hi)
            out[t, h] = attend(q[t, h], Kh, Vh, scale, softcap)
    return out
