"""The step loop bench.py times (allocator step into pinned memory, copies, fused append + table
patch + lengths, decode), run for 20 steps on a reduced Llama-shaped batch, against the oracle:
the final K/V pools, block tables and lengths are bit-identical to the oracle allocator's and
append's, and the last decode matches the oracle over that cache."""
import numpy as np
import pytest
import torch

import bench
import inputs
from oracle import cache_ops
from oracle.allocator import PyAllocator, run_script
from oracle.attention import decode_paged
from tests.gpu_cases import TOL, say

pytestmark = pytest.mark.gpu


def test_bench_step_loop_matches_oracle():
    w = inputs.small("llama8b_decode")
    steps = 20   # crosses block boundaries for several sequences
    say(f"bench step loop B={w.B} steps={steps}")
    r = bench.StepRunner(w, steps)
    for _ in range(steps):
        r.step()
    torch.cuda.synchronize()

    py = PyAllocator(w.NB, w.bs, inputs.free_order(w))
    ids = run_script(py, inputs.setup_script(w))
    seqs = [ids[b] for b in range(w.B)]
    pool = inputs.pool(w)
    k, v = pool["k"], pool["v"]
    for s in range(steps):
        slots, pairs = py.step(seqs)
        if pairs:
            k, v = cache_ops.copy_blocks(k, v, pairs)
        kn, vn = inputs.new_tokens(w, s)
        k, v = cache_ops.append(k, v, kn, vn, slots, w.bs)
    tables, lens = (np.asarray(x, np.int32) for x in py.export(seqs, r.MB))

    assert np.array_equal(r.k.view(torch.int16).cpu().numpy().view(np.uint16), k)
    assert np.array_equal(r.v.view(torch.int16).cpu().numpy().view(np.uint16), v)
    assert np.array_equal(r.tables.cpu().numpy(), tables)
    assert np.array_equal(r.lens_step.cpu().numpy(), lens)
    q = inputs.queries(w, (steps - 1) % len(r.q))
    ref = decode_paged(q, "bf16", k, v, "bf16", tables, lens, w.bs, w.scale)
    err = float(np.max(np.abs(r.out.cpu().numpy().astype(np.float64) - ref)))
    say(f"max-abs error {err:.2e}")
    assert err <= TOL["bf16"]
