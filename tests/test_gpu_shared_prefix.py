"""GPU parity of the shared-prefix decode (pa_decode_shared_prefix) against the fp64 oracle.

The shared-prefix decode computes the same attention as pa_decode; it only reads the blocks that
adjacent sequences share at the start of their tables once per group.  Its outputs are checked
against the oracle's plain per-sequence attention (max-abs within the decode tolerance of the
cache kind) and against pa_decode on the same inputs: both take each token's score and weight the
same way, so they agree far inside that tolerance (bf16 1e-4; the quantised kinds round
P * v_scale to fp16 relative to a different running maximum, 2^-12 of a value, hence 5e-3).

The batches are built from explicit block tables: groups whose members share a prefix of
full blocks, members shorter than, equal to and longer than their prefix, a partial last prefix
block that longer members hold a copy of, groups that cross the aligned windows of 64 sequences
the plan works in, more members than one 16-column tile holds, prefixes long enough to be split
into several parts, runs that share a first block and nothing more, lone and empty sequences,
and invalid table entries inside a shared prefix.
"""
import numpy as np
import pytest
import torch

import inputs
import paged_kv_cache_284_amd as pkv
from oracle import attention
from tests.gpu_cases import TOL, Case, max_err, poison_unused, sample_heads, say, to_device

pytestmark = pytest.mark.gpu

AGREE = {"bf16": 1e-4, "i8": 5e-3, "i4": 5e-3, "f32": 1e-5}


def _grouped(kv, G, D, groups, Hkv=2, cid=71, name="grouped"):
    """A decode-only batch from explicit tables.

    groups: list of (prefix, lengths).  The members of a group are adjacent in the batch and
    share the physical blocks of the first `prefix` tokens: a member with L <= prefix holds the
    first ceil(L / 16) of them; a longer one holds the prefix's full blocks, then (when the
    prefix ends inside a block) its own copy of that block, then private blocks.  Physical block
    numbers are a seeded permutation.  Returns (w, tables, lens, pool, q).
    """
    rows, lens = [], []
    nb = 0
    for prefix, Ls in groups:
        n_full, part = prefix // 16, prefix % 16
        shared = list(range(nb, nb + n_full + (1 if part else 0)))
        nb += len(shared)
        for L in Ls:
            if L <= prefix:
                row = shared[:(L + 15) // 16]
            else:
                row = shared[:n_full]
                rest = (L + 15) // 16 - len(row)
                row += list(range(nb, nb + rest))
                nb += rest
            rows.append(row)
            lens.append(L)
    NB = nb + 8
    perm = np.random.default_rng([cid, 9]).permutation(NB).astype(np.int32)
    B = len(lens)
    MB = max(1, max(len(r) for r in rows)) + 1
    tables = np.full((B, MB), -1, np.int32)
    for b, r in enumerate(rows):
        tables[b, :len(r)] = perm[r]
    lens = np.array(lens, np.int32)
    w = inputs.llama8b_decode(B=B, lo=1, hi=2, cid=cid, name=name)
    w.lengths = lens.astype(np.int64)
    w.Hkv, w.Hq, w.D, w.kv_dtype, w.q_dtype = Hkv, Hkv * G, D, kv, "bf16"
    w.NB = NB
    w.append = False
    pool = inputs.pool(w)
    poison_unused(pool, w, tables, lens)
    return w, tables, lens, pool, inputs.queries(w)


def _run(w, tables, lens, pool, q, both=True):
    dev = {k: (to_device(v, w.kv_dtype) if k in ("k", "v") else torch.from_numpy(v).cuda())
           for k, v in pool.items()}
    tab = torch.from_numpy(tables).cuda()
    ln = torch.from_numpy(lens).cuda()
    qd = to_device(q, "bf16")
    max_len = int(lens.max()) if len(lens) else 0
    ks, vs = dev.get("k_scale"), dev.get("v_scale")
    out = pkv.decode_shared_prefix(qd, dev["k"], dev["v"], tab, ln, max_len, w.scale, ks, vs)
    again = pkv.decode_shared_prefix(qd, dev["k"], dev["v"], tab, ln, max_len, w.scale, ks, vs)
    plain = pkv.decode(qd, dev["k"], dev["v"], tab, ln, max_len, w.scale, ks, vs) if both else None
    torch.cuda.synchronize()
    assert torch.equal(out, again), "repeated calls differ"
    return out.cpu().numpy(), None if plain is None else plain.cpu().numpy()


def _oracle(w, tables, lens, pool, q, heads=None):
    return attention.decode_paged(q, "bf16", pool["k"], pool["v"], w.kv_dtype, tables, lens, 16,
                                  w.scale, pool.get("k_scale"), pool.get("v_scale"), heads=heads)


def _check(kv, out, plain, ref):
    assert np.all(np.isfinite(out))
    err = max_err(out, ref)
    assert err <= TOL[kv], f"max-abs error against the oracle {err}"
    agree = float(np.max(np.abs(out - plain))) if out.size else 0.0
    assert agree <= AGREE[kv], f"differs from pa_decode by {agree}"


MIXED = [
    (1024, [300, 1500, 1025, 40, 1024, 2000, 17, 999]),  # lognormal-like members
    (96, [96, 96, 128, 64]),          # members that end at their prefix: nothing past it
    (40, [50, 60, 45]),               # the prefix ends inside a block: copies, 32 tokens shared
    (16, [20, 30, 40]),               # one shared block: below a pair, no prefix pass
    (0, [0]), (0, [1]), (0, [33]),    # an empty and lone sequences
    (200, [0, 180, 250]),             # an empty member splits the run
    (500, [700]),                     # a lone sequence whose blocks nobody shares
]


@pytest.mark.parametrize("kv,G,D", [("bf16", 4, 128), ("bf16", 1, 64), ("bf16", 2, 128),
                                    ("bf16", 8, 128), ("bf16", 8, 64), ("i8", 4, 128),
                                    ("i8", 1, 64), ("i4", 4, 128), ("i4", 8, 64)])
def test_mixed_groups(kv, G, D):
    w, tables, lens, pool, q = _grouped(kv, G, D, MIXED, cid=71 + G + D)
    say(f"shared-prefix mixed kv={kv} G={G} D={D} B={w.B}")
    out, plain = _run(w, tables, lens, pool, q)
    _check(kv, out, plain, _oracle(w, tables, lens, pool, q))
    for b in np.nonzero(lens == 0)[0]:  # empty sequences, lone and inside a run
        assert np.array_equal(out[b], np.zeros_like(out[b]))


@pytest.mark.parametrize("kv,G", [("bf16", 4), ("i8", 2)])
def test_group_across_windows(kv, G):
    """100 members of one prefix from batch entry 10 on: the plan's windows of 64 cut it into
    three groups, each reading the prefix once."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(150, 420, 100)]
    groups = [(0, [37 + i]) for i in range(10)] + [(200, lens), (0, [90])]
    w, tables, lens, pool, q = _grouped(kv, G, 128, groups, cid=90 + G)
    say(f"shared-prefix windows kv={kv} G={G} B={w.B}")
    out, plain = _run(w, tables, lens, pool, q)
    _check(kv, out, plain, _oracle(w, tables, lens, pool, q))


@pytest.mark.parametrize("kv,G,members", [("bf16", 8, 64), ("bf16", 1, 40), ("i4", 4, 20)])
def test_many_columns(kv, G, members):
    """More query columns (members x G) than one tile: several column blocks per KV head."""
    rng = np.random.default_rng(G + members)
    lens = [int(x) for x in rng.integers(100, 700, members)]
    w, tables, lens, pool, q = _grouped(kv, G, 128, [(512, lens)], cid=110 + G)
    say(f"shared-prefix columns kv={kv} G={G} members={members}")
    out, plain = _run(w, tables, lens, pool, q)
    _check(kv, out, plain, _oracle(w, tables, lens, pool, q))


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_long_prefix_in_parts(kv):
    """A prefix longer than one part of the prefix pass (parts of ~1.1 K tokens here): every
    member folds several prefix states."""
    groups = [(5000, [5000, 6010, 7000, 9000, 4700]), (3000, [3100, 3300]), (0, [8000])]
    w, tables, lens, pool, q = _grouped(kv, 4, 128, groups, cid=130)
    say(f"shared-prefix long kv={kv}")
    out, plain = _run(w, tables, lens, pool, q)
    _check(kv, out, plain, _oracle(w, tables, lens, pool, q))


def test_invalid_entry_inside_prefix():
    """A table entry outside [0, NB) inside the shared blocks: the plan stops sharing there and
    the result is pa_decode's (which skips that block's tokens)."""
    w, tables, lens, pool, q = _grouped("bf16", 4, 128, [(640, [700, 800, 900, 650])], cid=150)
    tables[:, 6] = w.NB + 3
    say("shared-prefix invalid entry")
    out, plain = _run(w, tables, lens, pool, q)
    assert np.all(np.isfinite(out))
    assert float(np.max(np.abs(out - plain))) <= AGREE["bf16"]


def test_first_block_only():
    """Sequences that share their first block and then diverge get no prefix pass: the outputs
    equal pa_decode's to rounding and the oracle's within tolerance."""
    w, tables, lens, pool, q = _grouped("bf16", 4, 128, [(16, [300, 310, 320, 16])], cid=160)
    out, plain = _run(w, tables, lens, pool, q)
    _check("bf16", out, plain, _oracle(w, tables, lens, pool, q))


@pytest.mark.parametrize("name", ["shared_prefix_batch", "llama8b_decode", "int8_mha",
                                  "int4_mha", "tiny_fp32"])
def test_small_workload_steps(name):
    """The small workloads through the whole step (allocator, copy-on-write, append), decoding
    with the shared-prefix call; fp32 falls back to pa_decode's schedule."""
    w = inputs.small(name)
    case = Case(w)
    for s in range(w.steps):
        say(f"{w.name} shared step {s}")
        q, out, tables, lens = case.step(shared=True)
        ref = case.oracle(q, tables, lens)
        assert np.all(np.isfinite(out))
        assert max_err(out, ref) <= TOL[w.kv_dtype], f"step {s}"
        assert float(np.max(np.abs(out - case.plain))) <= AGREE[w.kv_dtype], f"step {s}"


def test_full_shared_prefix_batch():
    """The full shared-prefix batch (B 256, groups of 8 sharing 1 K tokens) through all its
    steps, copy-on-write included: sampled rows against the oracle at the first and the last
    step, every row against pa_decode at every step."""
    w = inputs.full("shared_prefix_batch")
    case = Case(w, poison=True)
    for s in range(w.steps):
        check = s in (0, w.steps - 1)
        say(f"{w.name} full shared step {s}")
        q, out, tables, lens = case.step(check_pool=check, shared=True)
        assert np.all(np.isfinite(out))
        assert float(np.max(np.abs(out - case.plain))) <= AGREE["bf16"], f"step {s}"
        if check:
            heads = sample_heads(w, lens, 24, seed=s)
            ref = case.oracle(q, tables, lens, heads=heads)
            assert max_err(out, ref, heads) <= TOL["bf16"], f"step {s}"
