"""bench.py's command-line contract on the CPU: more than one GPU is refused with a
message (the library has no multi-GPU path), before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_byte_and_flop_models():
    """The algorithmic byte / flop counts bench.py reports, on small batches counted by
    hand: K and V once, Q and O, used table entries and lengths for decode; 4*D*H per
    visible (query, key) pair for prefill."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import bench
    from paged_kv_scaled_amd import workloads as wl
    lens = np.array([3, 17], np.int32)
    w = wl.build("hand", 0, "bf16", lens, np.ones(2, np.int32), 4, 2, 16, 4, wl.MASK_NONE,
                 decode=True)
    kv = 20 * 2 * 16 * 2 * 2          # keys x Hkv x D x 2 bytes x (K, V)
    qo = 2 * 2 * 4 * 16 * 2           # (Q, O) x seqs x H x D x 2 bytes
    tables = (1 + 5) * 4              # pages of 3 and 17 keys at B = 4
    assert bench.decode_bytes(w) == kv + qo + tables + 2 * 4
    w8 = wl.with_fp8_cache(wl.build("hand8", 0, "bf16", lens, np.ones(2, np.int32), 4, 2, 16, 4,
                                    wl.MASK_NONE, decode=True))
    assert bench.decode_bytes(w8) == kv // 2 + qo + tables + 2 * 4
    # causal prefill of one 5-token sequence: 15 visible pairs
    p = wl.build("handp", 0, "bf16", np.array([5], np.int32), np.array([5], np.int32), 4, 2, 16,
                 4, wl.MASK_CAUSAL)
    assert bench.prefill_flops(p) == 4.0 * 16 * 4 * 15
