"""Preemption by swapping on the GPU: sequences are swapped out to a pinned host pool with one
batched pa_swap_blocks launch, their device blocks are reused by other sequences, and they are
swapped back in; the device pool and the host pool match the oracle's copies bit-exactly after
every step, and decode over the swapped-in sequences matches the oracle."""
import numpy as np
import pytest
import torch

import inputs
import paged_kv_cache_284_amd as pkv
from oracle import attention, cache_ops
from oracle.allocator import run_script
from oracle.swap import SwappingAllocator
from tests.gpu_cases import TOL, from_device_bits, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["bf16", "i8", "i4"])
def test_swap_out_reuse_swap_in(kv):
    w = inputs.llama8b_decode(B=6, lo=20, hi=120, cid=85, name="swap")
    w.Hkv, w.Hq, w.D, w.append = 2, 8, 64, False
    w.kv_dtype = kv
    NCPU = 24
    w.NB = int(sum((L + 15) // 16 for L in w.lengths)) + 12
    order = inputs.free_order(w)
    lib = pkv.Allocator(w.NB, w.bs, order)
    lib.set_swap(NCPU)
    py = SwappingAllocator(w.NB, w.bs, order, num_cpu_blocks=NCPU)
    ops = inputs.setup_script(w)
    ids = pkv.run_script(lib, ops)
    assert run_script(py, ops) == ids
    seqs = [ids[b] for b in range(w.B)]
    host = inputs.pool(w)
    dev = {k: (to_device(v, kv) if k in ("k", "v") else torch.from_numpy(v).cuda())
           for k, v in host.items()}
    shape_k = (NCPU,) + host["k"].shape[1:]
    shape_v = (NCPU,) + host["v"].shape[1:]
    npdt = host["k"].dtype
    swap = {"k": np.zeros(shape_k, npdt), "v": np.zeros(shape_v, npdt)}
    tdt = {"bf16": torch.int16, "i8": torch.int8, "i4": torch.uint8}[kv]
    pin = {"k": torch.zeros(shape_k, dtype=tdt).pin_memory(),
           "v": torch.zeros(shape_v, dtype=tdt).pin_memory()}
    if kv == "bf16":
        pin = {k: t.view(torch.bfloat16) for k, t in pin.items()}
    if kv in ("i8", "i4"):
        for s in ("k_scale", "v_scale"):
            swap[s] = np.zeros((NCPU, w.Hkv), np.float32)
            pin[s] = torch.zeros((NCPU, w.Hkv), dtype=torch.float32).pin_memory()

    def scales(d):
        return (d.get("k_scale"), d.get("v_scale"))

    def check():
        torch.cuda.synchronize()
        for k in host:
            got = from_device_bits(dev[k]) if k in ("k", "v") else dev[k].cpu().numpy()
            assert np.array_equal(got.view(host[k].dtype), host[k]), k
        for k in swap:
            got = pin[k].view(torch.int16).numpy().view(np.uint16) if (kv == "bf16" and k in ("k", "v")) else pin[k].numpy()
            assert np.array_equal(got, swap[k]), k

    # swap out sequences 1 and 4
    out_pairs = {}
    for b in (1, 4):
        pl, pp = lib.swap_out(seqs[b]), py.swap_out(seqs[b])
        assert pl == pp
        out_pairs[b] = pp
        pairs = torch.tensor(pp, dtype=torch.int32).pin_memory()
        pkv.swap_blocks(dev["k"], dev["v"], pin["k"], pin["v"], pairs, scales(dev), scales(pin))
        for d, c in pp:
            for k in swap:
                swap[k][c] = host[k][d]
        say(f"{kv}: swapped out sequence {b}: {len(pp)} blocks")
    check()
    # other sequences take the released blocks and overwrite them
    if kv == "bf16":
        for b in (0, 2):
            n = 40
            slots_l, _ = lib.reserve(seqs[b], n)
            slots_p, _ = py.reserve(seqs[b], n)
            assert slots_l == slots_p
            kn, vn = inputs.token_kv(85, b, n, w.Hkv, w.D, kv)
            pkv.kv_append(to_device(kn, kv), to_device(vn, kv),
                          torch.tensor(slots_p, dtype=torch.int64, device="cuda"), dev["k"], dev["v"])
            host["k"], host["v"] = cache_ops.append(host["k"], host["v"], kn, vn, slots_p, w.bs)
        check()
    # swap back in (device blocks come from the free list: with the appends above, others)
    for b in (4, 1):
        pl, pp = lib.swap_in(seqs[b]), py.swap_in(seqs[b])
        assert pl == pp
        pairs = torch.tensor(pp, dtype=torch.int32, device="cuda")
        pkv.swap_blocks(pin["k"], pin["v"], dev["k"], dev["v"], pairs, scales(pin), scales(dev))
        for c, d in pp:
            for k in swap:
                host[k][d] = swap[k][c]
        say(f"{kv}: swapped in sequence {b}")
    check()
    tables, lens = py.export(seqs, 16)
    tables, lens = np.array(tables, np.int32), np.array(lens, np.int32)
    q = inputs.queries(w, 0)
    out = pkv.decode(to_device(q, "bf16"), dev["k"], dev["v"], torch.from_numpy(tables).cuda(),
                     torch.from_numpy(lens).cuda(), int(lens.max()), w.scale, *scales(dev))
    ref = attention.decode_paged(q, "bf16", host["k"], host["v"], kv, tables, lens, w.bs, w.scale,
                                 host.get("k_scale"), host.get("v_scale"))
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)))
    say(f"{kv}: decode after the round trip: max-abs error {err:.2e}")
    assert err <= TOL[kv]
