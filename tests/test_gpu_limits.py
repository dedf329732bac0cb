"""GPU parity at the decode schedules' size limits.

The balanced schedule keeps every sequence's pair count and cost in LDS, so it takes batches of
up to 8192 sequences (kMaxBalancedBatch); pa_decode with the automatic partition runs larger
batches on fixed partitions instead.  The shared-prefix plan works in aligned windows of 64
sequences, at most 128 of them, and its prefix pass keeps a record per group in LDS.  These
tests run each call at its largest batch and one past the balanced limit: sampled rows against
the fp64 oracle (within the decode tolerance) and every row against a second, differently
scheduled call on the same inputs (fixed partitions of 64 tokens), which sums the same products
in another order, so the two agree far inside the tolerance.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_284_amd as pkv
from tests.gpu_cases import TOL, max_err, say, to_device
from tests.test_gpu_shared_prefix import AGREE, _grouped, _oracle

pytestmark = pytest.mark.gpu

MAX_BALANCED = 8192


def _device(w, tables, lens, pool, q):
    dev = {k: (to_device(v, w.kv_dtype) if k in ("k", "v") else torch.from_numpy(v).cuda())
           for k, v in pool.items()}
    return (to_device(q, "bf16"), dev, torch.from_numpy(tables).cuda(),
            torch.from_numpy(lens).cuda(), int(lens.max()) if len(lens) else 0)


def _sampled(w, lens, n, seed):
    rng = np.random.default_rng(seed)
    picks = {(int(np.argmax(lens)), h) for h in range(w.Hq)}
    picks |= {(int(b), int(rng.integers(w.Hq))) for b in rng.integers(w.B, size=n)}
    picks |= {(int(b), 0) for b in np.nonzero(lens == 0)[0][:4]}
    return sorted(picks)


def _lone(n, rng, hi, zeros=8):
    """n sequences with private blocks, lengths U[1, hi] and a few empty ones."""
    L = [int(x) for x in rng.integers(1, hi + 1, n)]
    for i in rng.choice(n, zeros, replace=False):
        L[int(i)] = 0
    return [(0, [x]) for x in L]


@pytest.mark.parametrize("B,G,D", [(MAX_BALANCED, 4, 64), (MAX_BALANCED, 8, 128),
                                   (MAX_BALANCED + 1, 4, 64)])
def test_decode_at_the_balanced_limit(B, G, D):
    """B = 8192 runs the balanced schedule (G = 8, D = 128 is its largest LDS: the per-wave
    states beside the 2 B + 2 prefix sums), B = 8193 the fixed partitions the automatic
    partition picks; each against the oracle and against 64-token fixed partitions."""
    rng = np.random.default_rng(B + G)
    w, tables, lens, pool, q = _grouped("bf16", G, D, _lone(B, rng, 90), Hkv=1,
                                        cid=200 + (B + G) % 7, name="limit")
    say(f"limit decode B={B} G={G} D={D}")
    qd, dev, tab, ln, max_len = _device(w, tables, lens, pool, q)
    out = pkv.decode(qd, dev["k"], dev["v"], tab, ln, max_len, w.scale)
    other = pkv.decode(qd, dev["k"], dev["v"], tab, ln, max_len, w.scale, partition_tokens=64)
    torch.cuda.synchronize()
    out, other = out.cpu().numpy(), other.cpu().numpy()
    assert np.all(np.isfinite(out))
    assert float(np.max(np.abs(out - other))) <= AGREE["bf16"]
    for b in np.nonzero(lens == 0)[0]:
        assert np.array_equal(out[b], np.zeros_like(out[b]))
    heads = _sampled(w, lens, 48, B)
    ref = _oracle(w, tables, lens, pool, q, heads=heads)
    assert max_err(out, ref, heads) <= TOL["bf16"]


def test_shared_prefix_at_the_largest_batch():
    """8192 sequences in 128 windows: groups of 2 to 16 members sharing 16 to 96 tokens (some
    crossing a window boundary), lone and empty sequences between them."""
    rng = np.random.default_rng(8192)
    groups, n = [], 0
    while n < MAX_BALANCED:
        if rng.random() < 0.3:
            spec = (0, [int(rng.integers(0, 60))])
        else:
            m = int(rng.integers(2, 17))
            prefix = 16 * int(rng.integers(1, 7))
            spec = (prefix, [int(x) for x in rng.integers(1, prefix + 40, m)])
        spec = (spec[0], spec[1][:MAX_BALANCED - n])
        groups.append(spec)
        n += len(spec[1])
    w, tables, lens, pool, q = _grouped("bf16", 4, 64, groups, Hkv=1, cid=209, name="limit")
    assert w.B == MAX_BALANCED
    say(f"limit shared-prefix B={w.B} groups={len(groups)}")
    qd, dev, tab, ln, max_len = _device(w, tables, lens, pool, q)
    out = pkv.decode_shared_prefix(qd, dev["k"], dev["v"], tab, ln, max_len, w.scale)
    plain = pkv.decode(qd, dev["k"], dev["v"], tab, ln, max_len, w.scale)
    torch.cuda.synchronize()
    out, plain = out.cpu().numpy(), plain.cpu().numpy()
    assert np.all(np.isfinite(out))
    assert float(np.max(np.abs(out - plain))) <= AGREE["bf16"]
    heads = _sampled(w, lens, 48, 1)
    ref = _oracle(w, tables, lens, pool, q, heads=heads)
    assert max_err(out, ref, heads) <= TOL["bf16"]
