"""bench.py's byte and flop accounting, checked by hand on tiny cases (CPU only)."""
import numpy as np

import bench
import inputs


def _w(kv="bf16", B=2, Hq=4, Hkv=2, D=64):
    w = inputs.tiny_fp32()
    w.kv_dtype, w.q_dtype, w.B, w.Hq, w.Hkv, w.D = kv, "bf16", B, Hq, Hkv, D
    return w


def test_shared_block_counts_once():
    w = _w()
    lens = np.array([20, 18])
    tables = np.array([[5, 7], [5, 9]])     # block 5 shared in full, 7 and 9 private
    per_token = w.Hkv * w.D * 2 * 2         # K and V, bf16
    fixed = w.B * w.Hq * w.D * 2 + w.B * w.Hq * w.D * 4 + 4 * 4 + w.B * 4  # q, out, 4 table entries, lens
    assert bench.algorithmic_bytes(w, lens) == 38 * per_token + fixed
    assert bench.algorithmic_bytes(w, lens, tables) == (16 + 4 + 2) * per_token + fixed


def test_partially_shared_block_takes_its_longest_reader():
    w = _w(kv="i8")
    lens = np.array([10, 13])
    tables = np.array([[3], [3]])           # one block read to 10 and to 13 tokens
    per_token = w.Hkv * w.D * 2 * 1
    fixed = w.B * w.Hq * w.D * 2 + w.B * w.Hq * w.D * 4 + 2 * 4 + w.B * 4
    scales = 1 * w.Hkv * 2 * 4               # one touched tile per KV head, K and V scales
    assert bench.algorithmic_bytes(w, lens, tables) == 13 * per_token + scales + fixed


def test_prefill_flops_brute_force():
    w = _w(Hq=4, D=64)
    lens, chunks = [7, 5, 3], [3, 5, 1]
    keys = 0
    for L, n in zip(lens, chunks):
        for i in range(n):
            keys += (L - n + i) + 1          # keys 0..p of the query at position p
    assert bench.prefill_flops(w, lens, chunks) == 4 * w.D * w.Hq * keys


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    """bench.py measures one GPU: --gpus 2 (or a multi-rank launch) exits with status 2 and says
    why, without importing torch."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args],
                           capture_output=True, text=True, timeout=120,
                           env={**os.environ, **env})
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def test_prefix_cache_measurement_reuses_the_shared_prompt(capsys):
    """The host prefix-cache measurement (no GPU work): every request finds the 3,000-token
    prompt's 187 full blocks cached (2,992 tokens, the page's example), never its private
    tokens, and the line reports what it timed."""
    import json
    import types
    bench.run_prefix_cache(types.SimpleNamespace(steps=3, warmup=1))
    r = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert r["cached_tokens_per_request"] == 2992
    assert r["config"]["requests_per_step"] == 64 and r["steps"] == 3
    assert r["value"] > 0 and r["us_per_request"] > 0
    assert abs(r["value"] * r["us_per_request"] - 1e6) < 1e-2 * 1e6
