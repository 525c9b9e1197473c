"""ctypes binding of libg4attn.so: argument marshalling only.

Every function here has the name of the C entry point it calls (declared in
include/g4attn.h) and does nothing but convert Python ints / torch tensors to
pointers and sizes and turn a negative status into ``G4AttnError``.  All
arithmetic runs in the library's HIP kernels; there is no Python fallback:
if the library is missing, ``load()`` raises.

``Stack`` is a small convenience owner of one layer stack: it keeps the
host-side plan handle and the device cache / workspace tensors that PyTorch
allocates, and checks tensor shapes before calling the entry points.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_float, c_int32, c_int64, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libg4attn.so")

G4ATTN_OK = 0
G4ATTN_ERR_NULL = -1
G4ATTN_ERR_DESC = -2
G4ATTN_ERR_OWNER = -3
G4ATTN_ERR_SHARED_LAYER = -4
G4ATTN_ERR_RANGE = -5
G4ATTN_ERR_UNBOUND = -6
G4ATTN_ERR_UNSUPPORTED = -7
G4ATTN_ERR_HIP = -8

ERROR_NAMES = {
    G4ATTN_ERR_NULL: "G4ATTN_ERR_NULL",
    G4ATTN_ERR_DESC: "G4ATTN_ERR_DESC",
    G4ATTN_ERR_OWNER: "G4ATTN_ERR_OWNER",
    G4ATTN_ERR_SHARED_LAYER: "G4ATTN_ERR_SHARED_LAYER",
    G4ATTN_ERR_RANGE: "G4ATTN_ERR_RANGE",
    G4ATTN_ERR_UNBOUND: "G4ATTN_ERR_UNBOUND",
    G4ATTN_ERR_UNSUPPORTED: "G4ATTN_ERR_UNSUPPORTED",
    G4ATTN_ERR_HIP: "G4ATTN_ERR_HIP",
}

# Entry points declared in include/g4attn.h, with (restype, argtypes).
_SIGNATURES = {
    "g4attn_stack_create": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32,
                                      POINTER(c_void_p)]),
    "g4attn_stack_destroy": (None, [c_void_p]),
    "g4attn_cache_bytes": (c_int32, [c_void_p, POINTER(c_uint64)]),
    "g4attn_workspace_bytes": (c_int32, [c_void_p, POINTER(c_uint64)]),
    "g4attn_bind": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "g4attn_resolve_owner": (c_int32, [c_void_p, c_int32, POINTER(c_int32)]),
    "g4attn_layer_capacity": (c_int32, [c_void_p, c_int32, POINTER(c_int32)]),
    "g4attn_key_range": (c_int32, [c_void_p, c_int32, c_int64, c_int64, POINTER(c_int64),
                                   POINTER(c_int64)]),
    "g4attn_kv_offset": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int64, c_int32,
                                   POINTER(c_int64), POINTER(c_int64)]),
    "g4attn_append_kv": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_int32, c_int32, c_int32, c_void_p]),
    "g4attn_decode": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                c_void_p, c_void_p]),
    "g4attn_decode_noalloc": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                        c_void_p, c_void_p]),
    "g4attn_decode_append": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
    "g4attn_prefill": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                 c_int32, c_void_p, c_void_p]),
    "g4attn_stack_create_paged": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32,
                                            c_int32, c_int32, POINTER(c_void_p)]),
    "g4attn_page_offset": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                     POINTER(c_int64), POINTER(c_int64)]),
    "g4attn_append_kv_paged": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                         c_void_p]),
    "g4attn_decode_paged": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                      c_void_p, c_void_p, c_void_p]),
    "g4attn_prefill_paged": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                       c_int32, c_void_p, c_void_p, c_void_p]),
    "g4attn_decode_append_paged": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                             c_void_p]),
    "g4attn_last_error": (ctypes.c_char_p, []),
}


class LayerDescC(ctypes.Structure):
    """Mirror of g4attn_layer_desc."""

    _fields_ = [
        ("n_q_heads", c_int32),
        ("n_kv_heads", c_int32),
        ("head_dim", c_int32),
        ("window", c_int32),
        ("k_eq_v", c_int32),
        ("kv_owner_layer", c_int32),
        ("scale", c_float),
        ("softcap", c_float),
    ]


class G4AttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code


_lib = None


def load():
    """Load libg4attn.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        try:  # share torch's HIP runtime (same soname) when torch is present
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != G4ATTN_OK:
        raise G4AttnError(rc, load().g4attn_last_error().decode())


def _ptr(x):
    """Device pointer of a tensor, or an int / None passed through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("tensors passed to g4attn must be contiguous")
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


def layer_descs(layers) -> ctypes.Array:
    arr = (LayerDescC * len(layers))()
    for i, d in enumerate(layers):
        arr[i] = LayerDescC(d.n_q_heads, d.n_kv_heads, d.head_dim, d.window, d.k_eq_v,
                            d.kv_owner_layer, d.scale, getattr(d, "softcap", 0.0))
    return arr


# ---------------------------------------------------------------------------
# one wrapper per C entry point
# ---------------------------------------------------------------------------

def g4attn_stack_create(layers, max_batch: int, kv_max: int, max_chunk: int) -> int:
    arr = layer_descs(layers)
    out = c_void_p()
    _check(load().g4attn_stack_create(ctypes.cast(arr, c_void_p), len(layers), max_batch, kv_max,
                                      max_chunk, byref(out)))
    return out.value


def g4attn_stack_destroy(stack: int) -> None:
    load().g4attn_stack_destroy(stack)


def g4attn_cache_bytes(stack: int) -> int:
    v = c_uint64()
    _check(load().g4attn_cache_bytes(stack, byref(v)))
    return v.value


def g4attn_workspace_bytes(stack: int) -> int:
    v = c_uint64()
    _check(load().g4attn_workspace_bytes(stack, byref(v)))
    return v.value


def g4attn_bind(stack: int, cache, workspace) -> None:
    _check(load().g4attn_bind(stack, _ptr(cache), _ptr(workspace)))


def g4attn_resolve_owner(stack: int, layer: int) -> int:
    v = c_int32()
    _check(load().g4attn_resolve_owner(stack, layer, byref(v)))
    return v.value


def g4attn_layer_capacity(stack: int, layer: int) -> int:
    v = c_int32()
    _check(load().g4attn_layer_capacity(stack, layer, byref(v)))
    return v.value


def g4attn_key_range(stack: int, layer: int, q_pos: int, n_keys: int) -> tuple[int, int]:
    lo, hi = c_int64(), c_int64()
    _check(load().g4attn_key_range(stack, layer, q_pos, n_keys, byref(lo), byref(hi)))
    return lo.value, hi.value


def g4attn_kv_offset(stack: int, layer: int, b: int, kv_head: int, pos: int,
                     d: int) -> tuple[int, int]:
    ok_, ov = c_int64(), c_int64()
    _check(load().g4attn_kv_offset(stack, layer, b, kv_head, pos, d, byref(ok_), byref(ov)))
    return ok_.value, ov.value


def g4attn_append_kv(stack: int, layer: int, k, v, start_pos, n_valid, batch: int, n_new: int,
                     max_end_pos: int, stream=None) -> None:
    _check(load().g4attn_append_kv(stack, layer, _ptr(k), _ptr(v), _ptr(start_pos),
                                   _ptr(n_valid), batch, n_new, max_end_pos, _stream(stream)))


def g4attn_decode(stack: int, layer: int, q, seq_lens, batch: int, max_seq_len: int, out,
                  stream=None) -> None:
    _check(load().g4attn_decode(stack, layer, _ptr(q), _ptr(seq_lens), batch, max_seq_len,
                                _ptr(out), _stream(stream)))


def g4attn_decode_noalloc(stack: int, layer: int, q, seq_lens, batch: int, max_seq_len: int,
                          out, stream=None) -> None:
    _check(load().g4attn_decode_noalloc(stack, layer, _ptr(q), _ptr(seq_lens), batch,
                                        max_seq_len, _ptr(out), _stream(stream)))


def g4attn_decode_append(stack: int, layer: int, q, k_new, v_new, seq_lens, batch: int,
                         max_seq_len: int, out, stream=None) -> None:
    _check(load().g4attn_decode_append(stack, layer, _ptr(q), _ptr(k_new), _ptr(v_new),
                                       _ptr(seq_lens), batch, max_seq_len, _ptr(out),
                                       _stream(stream)))


def g4attn_prefill(stack: int, layer: int, q, start_pos, batch: int, n_tok: int,
                   max_start_pos: int, out, stream=None) -> None:
    _check(load().g4attn_prefill(stack, layer, _ptr(q), _ptr(start_pos), batch, n_tok,
                                 max_start_pos, _ptr(out), _stream(stream)))


def g4attn_stack_create_paged(layers, max_batch: int, page_size: int, n_pages: int,
                              max_pages_per_seq: int, max_chunk: int) -> int:
    arr = layer_descs(layers)
    out = c_void_p()
    _check(load().g4attn_stack_create_paged(ctypes.cast(arr, c_void_p), len(layers), max_batch,
                                            page_size, n_pages, max_pages_per_seq, max_chunk,
                                            byref(out)))
    return out.value


def g4attn_page_offset(stack: int, layer: int, page: int, kv_head: int, slot: int,
                       d: int) -> tuple[int, int]:
    ok_, ov = c_int64(), c_int64()
    _check(load().g4attn_page_offset(stack, layer, page, kv_head, slot, d, byref(ok_), byref(ov)))
    return ok_.value, ov.value


def g4attn_append_kv_paged(stack: int, layer: int, k, v, start_pos, n_valid, batch: int,
                           n_new: int, max_end_pos: int, block_table, stream=None) -> None:
    _check(load().g4attn_append_kv_paged(stack, layer, _ptr(k), _ptr(v), _ptr(start_pos),
                                         _ptr(n_valid), batch, n_new, max_end_pos,
                                         _ptr(block_table), _stream(stream)))


def g4attn_decode_paged(stack: int, layer: int, q, seq_lens, batch: int, max_seq_len: int,
                        block_table, out, stream=None) -> None:
    _check(load().g4attn_decode_paged(stack, layer, _ptr(q), _ptr(seq_lens), batch, max_seq_len,
                                      _ptr(block_table), _ptr(out), _stream(stream)))


def g4attn_decode_append_paged(stack: int, layer: int, q, k_new, v_new, seq_lens, batch: int,
                               max_seq_len: int, block_table, out, stream=None) -> None:
    _check(load().g4attn_decode_append_paged(stack, layer, _ptr(q), _ptr(k_new), _ptr(v_new),
                                             _ptr(seq_lens), batch, max_seq_len,
                                             _ptr(block_table), _ptr(out), _stream(stream)))


def g4attn_prefill_paged(stack: int, layer: int, q, start_pos, batch: int, n_tok: int,
                         max_start_pos: int, block_table, out, stream=None) -> None:
    _check(load().g4attn_prefill_paged(stack, layer, _ptr(q), _ptr(start_pos), batch, n_tok,
                                       max_start_pos, _ptr(block_table), _ptr(out),
                                       _stream(stream)))


def g4attn_last_error() -> str:
    return load().g4attn_last_error().decode()


# ---------------------------------------------------------------------------
# convenience owner of a stack and its device buffers
# ---------------------------------------------------------------------------

class Stack:
    """A planned layer stack with its cache and workspace on a torch device."""

    def __init__(self, layers, max_batch: int, kv_max: int, max_chunk: int = 64,
                 device="cuda", page_size=None, n_pages=None):
        """page_size / n_pages: a paged cache (kv_max a multiple of page_size); its
        calls then go through `block_table`, an int32 [max_batch, kv_max // page_size]
        device tensor of page ids that the caller sets."""
        import torch

        self.layers = list(layers)
        self.max_batch, self.kv_max, self.max_chunk = max_batch, kv_max, max_chunk
        self.paged = page_size is not None
        self.block_table = None
        if self.paged:
            if kv_max % page_size:
                raise ValueError("kv_max must be a multiple of page_size")
            self.page_size, self.n_pages = page_size, n_pages
            self.max_pages = kv_max // page_size
            self.handle = g4attn_stack_create_paged(self.layers, max_batch, page_size, n_pages,
                                                    self.max_pages, max_chunk)
        else:
            self.handle = g4attn_stack_create(self.layers, max_batch, kv_max, max_chunk)
        self.cache_nbytes = g4attn_cache_bytes(self.handle)
        self.ws_nbytes = g4attn_workspace_bytes(self.handle)
        self.device = torch.device(device)
        self.cache = torch.zeros(max(self.cache_nbytes, 256), dtype=torch.uint8,
                                 device=self.device)
        self.workspace = torch.zeros(max(self.ws_nbytes, 256), dtype=torch.uint8,
                                     device=self.device)
        # the zero fill runs on torch's current stream; the library's calls may
        # go to any stream, so finish it before the first of them
        if self.device.type == "cuda":
            torch.cuda.synchronize(self.device)
        g4attn_bind(self.handle, self.cache, self.workspace)

    def close(self):
        if getattr(self, "handle", None):
            g4attn_stack_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _table(self):
        import torch

        if self.block_table is None:
            raise ValueError("a paged stack needs its block_table set")
        _expect(self.block_table, (self.max_batch, self.max_pages), torch.int32, "block_table")
        return self.block_table

    def owner(self, layer: int) -> int:
        return g4attn_resolve_owner(self.handle, layer)

    def capacity(self, layer: int) -> int:
        return g4attn_layer_capacity(self.handle, layer)

    def append_kv(self, layer, k, v, start_pos, n_valid=None, max_end_pos=None, stream=None):
        """k, v: bf16 [B, T, n_kv, D]; start_pos / n_valid: int32 [B] on the device."""
        import torch

        d = self.layers[layer]
        B, T = k.shape[0], k.shape[1]
        _expect(k, (B, T, d.n_kv_heads, d.head_dim), torch.bfloat16, "k")
        if v is not None:
            _expect(v, (B, T, d.n_kv_heads, d.head_dim), torch.bfloat16, "v")
        _expect(start_pos, (B,), torch.int32, "start_pos")
        if n_valid is not None:
            _expect(n_valid, (B,), torch.int32, "n_valid")
        if max_end_pos is None:
            raise ValueError("max_end_pos (host bound on start_pos + n_valid) is required")
        if self.paged:
            g4attn_append_kv_paged(self.handle, layer, k, v, start_pos, n_valid, B, T,
                                   max_end_pos, self._table(), stream)
        else:
            g4attn_append_kv(self.handle, layer, k, v, start_pos, n_valid, B, T, max_end_pos,
                             stream)

    def decode(self, layer, q, seq_lens, max_seq_len, out=None, stream=None):
        """q: bf16 [B, n_q, D]; seq_lens: int32 [B] (keys incl. the current one)."""
        import torch

        d = self.layers[layer]
        B = q.shape[0]
        _expect(q, (B, d.n_q_heads, d.head_dim), torch.bfloat16, "q")
        _expect(seq_lens, (B,), torch.int32, "seq_lens")
        if out is None:
            out = torch.empty_like(q)
        _expect(out, tuple(q.shape), torch.bfloat16, "out")
        if self.paged:
            g4attn_decode_paged(self.handle, layer, q, seq_lens, B, max_seq_len, self._table(),
                                out, stream)
        else:
            g4attn_decode(self.handle, layer, q, seq_lens, B, max_seq_len, out, stream)
        return out

    def decode_append(self, layer, q, k_new, v_new, seq_lens, max_seq_len, out=None,
                      stream=None):
        """Decode with the current token's K/V written first. q: bf16 [B, n_q, D];
        k_new, v_new: bf16 [B, n_kv, D] (v_new None on k_eq_v layers);
        seq_lens: int32 [B] (keys incl. the current one)."""
        import torch

        d = self.layers[layer]
        B = q.shape[0]
        _expect(q, (B, d.n_q_heads, d.head_dim), torch.bfloat16, "q")
        _expect(k_new, (B, d.n_kv_heads, d.head_dim), torch.bfloat16, "k_new")
        if v_new is not None:
            _expect(v_new, (B, d.n_kv_heads, d.head_dim), torch.bfloat16, "v_new")
        _expect(seq_lens, (B,), torch.int32, "seq_lens")
        if out is None:
            out = torch.empty_like(q)
        _expect(out, tuple(q.shape), torch.bfloat16, "out")
        if self.paged:
            g4attn_decode_append_paged(self.handle, layer, q, k_new, v_new, seq_lens, B,
                                       max_seq_len, self._table(), out, stream)
        else:
            g4attn_decode_append(self.handle, layer, q, k_new, v_new, seq_lens, B, max_seq_len,
                                 out, stream)
        return out

    def prefill(self, layer, q, start_pos, max_start_pos, out=None, stream=None):
        """q: bf16 [B, T, n_q, D]; start_pos: int32 [B]."""
        import torch

        d = self.layers[layer]
        B, T = q.shape[0], q.shape[1]
        _expect(q, (B, T, d.n_q_heads, d.head_dim), torch.bfloat16, "q")
        _expect(start_pos, (B,), torch.int32, "start_pos")
        if out is None:
            out = torch.empty_like(q)
        _expect(out, tuple(q.shape), torch.bfloat16, "out")
        if self.paged:
            g4attn_prefill_paged(self.handle, layer, q, start_pos, B, T, max_start_pos,
                                 self._table(), out, stream)
        else:
            g4attn_prefill(self.handle, layer, q, start_pos, B, T, max_start_pos, out, stream)
        return out


def _expect(t, shape, dtype, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
