"""CPU checks of the benchmark's contract: it refuses more than one GPU, its
algorithmic byte and flop counts equal closed forms of the workloads, and the
HBM traffic it reports comes only from counters taken on the kernel source
that is built."""

import os
import subprocess
import sys

import bench
from decode_attention_gemma_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_decode_kv_bytes_closed_form():
    # 40 sliding layers: 16 sequences x 8 KV heads x 1024 visible keys (every
    # context is >= 1024) x 256 dims x 2 bytes x (K, V); 8 global k_eq_v
    # layers: every cached key once, 512 dims x 2 bytes
    wl = W.g12b_decode()
    assert min(wl.seq_lens) >= 1024
    want = 40 * 16 * 8 * 1024 * 256 * 2 * 2 + 8 * sum(wl.seq_lens) * 512 * 2
    assert sum(bench.kv_bytes(wl, i) for i in range(wl.n_layers)) == want == 5708152832


def test_prefill_flops_closed_form():
    # prefix 4032: a sliding token sees exactly 1024 keys; global token t sees
    # 4033 + t keys; 4 x head_dim flops per (query head, key) pair
    wl = W.g12b_prefill(4032)
    sliding = 40 * 4 * 64 * 16 * 1024 * 4 * 256
    glob = 8 * 4 * 16 * sum(4033 + t for t in range(64)) * 4 * 512
    assert sum(bench.prefill_flops(wl, i) for i in range(wl.n_layers)) == sliding + glob
    # prefix 0: causal within the chunk, token t sees t + 1 keys on every layer
    wl0 = W.g12b_prefill(0)
    tri = sum(t + 1 for t in range(64))
    want0 = 40 * 4 * 16 * tri * 4 * 256 + 8 * 4 * 16 * tri * 4 * 512
    assert sum(bench.prefill_flops(wl0, i) for i in range(wl0.n_layers)) == want0


def test_prefill_kv_bytes_closed_form():
    # prefix 4032: a sliding (sequence, KV head) reads keys 3009 .. 4095
    # (1087 keys, K and V); a global one reads all 4096 keys once (k_eq_v)
    wl = W.g12b_prefill(4032)
    assert bench.prefill_kv_bytes(wl, 0) == 4 * 8 * 1087 * 256 * 2 * 2
    assert bench.prefill_kv_bytes(wl, 5) == 4 * 1 * 4096 * 512 * 2


def test_counter_traffic_only_for_the_profiled_source(tmp_path, monkeypatch):
    got = bench.counter_traffic(bench.DOMINANT_KERNEL)
    text = open(bench.COUNTER_SUMMARY).read()
    hashes = bench.source_hashes()
    if all(f"{n} sha256[:16]: {h}" in text for n, h in hashes.items()):
        assert got is not None and got > 0
    else:
        assert got is None
    for attr, name in (("KERNEL_SOURCE", "kernels.hip"), ("PLAN_SOURCE", "plan.cpp")):
        other = tmp_path / name
        other.write_bytes(open(getattr(bench, attr), "rb").read() + b"\n// edited\n")
        monkeypatch.setattr(bench, attr, str(other))
        assert bench.counter_traffic(bench.DOMINANT_KERNEL) is None
        monkeypatch.undo()


def test_probe_library_exports_its_entry_points():
    """The hardware-rate probes bench.py --read-probe / --gemm-probe /
    --delivery-probe time are built beside the library and export their C
    entry points (no GPU call here)."""
    import ctypes

    from decode_attention_gemma_amd import build as B

    if not os.path.exists(B.PROBE_LIB):
        import pytest

        pytest.skip("libg4probe.so not built")
    lib = ctypes.CDLL(B.PROBE_LIB)
    names = ("g4probe_read", "g4probe_mfma", "g4probe_lds", "g4probe_l2")
    assert all(hasattr(lib, n) for n in names)
    # the attention library's ABI does not carry them
    from decode_attention_gemma_amd import g4attn

    main = ctypes.CDLL(g4attn.LIB_PATH)
    assert not any(hasattr(main, n) for n in names)
