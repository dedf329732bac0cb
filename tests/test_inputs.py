"""The seeded input generators: determinism, shapes and ranges of each workload, bf16 rounding
against torch's CPU cast, and the int8 quantiser's bounds."""
import hashlib

import numpy as np
import pytest
import torch

import inputs


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("name", ["tiny_fp32", "llama8b_decode", "long_context",
                                  "shared_prefix_batch", "int8_mha"])
def test_small_workloads_are_deterministic(name):
    a, b = inputs.small(name), inputs.small(name)
    pa, pb = inputs.pool(a), inputs.pool(b)
    assert _digest(a.lengths, inputs.free_order(a), inputs.queries(a), *pa.values()) == \
        _digest(b.lengths, inputs.free_order(b), inputs.queries(b), *pb.values())


def test_full_workload_shapes():
    w = inputs.tiny_fp32()
    assert list(w.lengths) == [1, 16, 17, 100] and w.NB == 64 and w.G == 2 and w.D == 64
    assert list(w.cached_lengths) == [0, 15, 16, 99]
    w = inputs.llama8b_decode()
    assert w.B == 64 and w.Hq == 32 and w.Hkv == 8 and w.D == 128
    assert 512 <= w.lengths.min() and w.lengths.max() <= 4096
    need = int(((w.lengths - 1 + 15) // 16).sum())
    assert w.NB >= 1.1 * need
    w = inputs.long_context()
    assert list(w.lengths) == [8192, 32768, 65536, 131072]
    w = inputs.shared_prefix_batch()
    assert w.B == 256 and w.group == 8 and w.prefix_tokens == 1024 and w.steps == 16
    assert 1 <= w.lengths.min() and w.lengths.max() <= 8192
    assert 600 < float(np.median(w.lengths)) < 1600
    w = inputs.int8_mha()
    assert w.B == 32 and w.Hq == w.Hkv == 40 and not w.append
    assert 1 <= w.lengths.min() and w.lengths.max() <= 2048


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100_000).astype(np.float32)
    ties = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 2**-130, 0.0, -0.0, 3e38],
                    np.float32)
    x = np.concatenate([x, ties, x * 1e-30, x * 1e30])
    ours = inputs.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(inputs.bf16_bits_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_int8_quantiser_bounds():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 3, 16, 8)).astype(np.float32)
    x[4, 1] = 0.0
    codes, scale = inputs.quantize_int8_pool(x)
    assert codes.dtype == np.int8 and scale.shape == (9, 3)
    assert codes.min() >= -127 and codes.max() <= 127
    assert scale[4, 1] == 1.0 and not codes[4, 1].any()
    for b in range(9):
        for g in range(3):
            if b == 4 and g == 1:
                continue
            t = x[b, g]
            i = np.unravel_index(np.argmax(np.abs(t)), t.shape)
            assert abs(int(codes[b, g][i])) == 127
            err = np.abs(t.astype(np.float64) - codes[b, g] * np.float64(scale[b, g]))
            assert err.max() <= scale[b, g] / 2 * (1 + 1e-6)


def test_peak_fraction_is_about_one_percent():
    w = inputs.small("long_context")
    k, _ = inputs.pool_f32(w)
    big = np.abs(k).max(axis=(1, 3)) > 6.0          # [NB][bs]
    frac = big.mean()
    assert 0.005 < frac < 0.02


def test_setup_script_plain_and_grouped():
    w = inputs.small("llama8b_decode")
    ops = inputs.setup_script(w)
    assert ops[:2] == [("create", 0), ("reserve", 0, int(w.cached_lengths[0]))]
    w = inputs.small("shared_prefix_batch")
    ops = inputs.setup_script(w)
    assert ops[0][0] == "create" and ops[0][1] == w.B
    assert sum(1 for o in ops if o[0] == "fork") == w.B
    assert sum(1 for o in ops if o[0] == "free") == w.B // w.group
