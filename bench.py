#!/usr/bin/env python3
"""Decode-step benchmark for the paged KV cache on one MI355X.

One step is one pass of the whole hot path over the batch:
  host allocator step (slot of each new token, lengths, table changes, copy-on-write pairs)
  written straight into pinned memory, where the kernels read them
  -> copy_blocks (only when a copy-on-write arose) -> fused append + block-table patch + length
  copy -> decode (+ merge of split segments).
Inputs (pools, queries, new tokens) are resident in HBM before the timed region starts.

Prints one JSON line: whole-job tokens/s (B decode tokens per step), the decode kernel's achieved
HBM GB/s against the MI355X peak (algorithmic bytes / mean launch time from HIP events on the
launch stream), and the CPU oracle timed on the host cores.  Algorithmic bytes count a block
that several sequences share once (unique bytes); the per-sequence sum is reported beside them.
Also reported: the append's time per step (copy-on-write copies included), the decode timed
alone after reading 1 GiB of other memory (cold caches), a plain device copy's rate for context,
and the oracle on all host threads.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--settle-ms 300]
                    [--workload llama8b_decode]

Before the warm-up steps, untimed decode calls on the first step's state (fixed partitions of
8192 tokens; they change no state) run for --settle-ms, so that timing starts with the GPU in
the state it holds under sustained decoding.

--workload prefill_llama8b measures the chunked-prefill path instead: one step appends a
512-token chunk per sequence (one pa_kv_append entry per token) and runs pa_prefill over it;
the roofline is then the matrix cores' bf16 peak (fp16 for the int8 / int4 caches of
prefill_llama8b_i8 / prefill_llama8b_i4, the same 2.5 PFLOP/s).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0   # dense MFMA bf16
METRIC = "paged decode attn: tokens/s + achieved HBM GB/s (% of MI355X peak)"
KV_BYTES = {"f32": 4, "bf16": 2, "i8": 1, "i4": 0.5}


def algorithmic_bytes(w, lens, tables=None) -> int:
    """Bytes a decode launch must move at minimum: K/V of every cached token, the int8 / int4
    scales of every touched (block, KV head) tile, q, out, the table entries in use and the
    lengths.  With the block tables given, a physical block that several sequences share counts
    once, with as many tokens as its longest user reads (the unique bytes)."""
    lens = np.asarray(lens, np.int64)
    blocks = (lens + w.bs - 1) // w.bs
    per_token = w.Hkv * w.D * 2 * KV_BYTES[w.kv_dtype]
    if tables is None:
        tokens, touched = int(lens.sum()), int(blocks.sum())
    else:
        used = {}
        for b in range(w.B):
            for j in range(int(blocks[b])):
                blk = int(tables[b][j])
                used[blk] = max(used.get(blk, 0), int(min(w.bs, lens[b] - j * w.bs)))
        tokens, touched = sum(used.values()), len(used)
    kv = int(tokens * per_token)
    scales = touched * w.Hkv * 2 * 4 if w.kv_dtype in ("i8", "i4") else 0
    q = w.B * w.Hq * w.D * KV_BYTES[w.q_dtype]
    out = w.B * w.Hq * w.D * 4
    return kv + scales + q + out + int(blocks.sum()) * 4 + w.B * 4


class HipEvents:
    """HIP events created with hipEventDisableSystemFence: recording them costs no system-scope
    cache writeback / invalidation, so they time the stream without stretching it (a default
    event adds a ~6 us bubble before the next launch on MI355X)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes as C
        self.C = C
        self.hip = C.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
        self.hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        e = self.C.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.C.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def record(self, e, stream):
        if self.hip.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def sync(self, e):
        if self.hip.hipEventSynchronize(e) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def elapsed_ms(self, e0, e1) -> float:
        ms = self.C.c_float()
        if self.hip.hipEventElapsedTime(self.C.byref(ms), e0, e1) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def build_workload(name: str, total_steps: int):
    import inputs
    if name == "llama8b_decode":
        return inputs.llama8b_decode(steps=total_steps)
    if name == "llama8b_decode_tp8":
        return inputs.llama8b_decode_tp8(steps=total_steps)
    if name == "shared_prefix_batch":
        return inputs.shared_prefix_batch(steps=total_steps)
    if name == "long_context":
        return inputs.long_context()
    if name == "int8_mha":
        return inputs.int8_mha()
    if name == "int4_mha":
        return inputs.int4_mha()
    if name == "tiny_fp32":
        return inputs.tiny_fp32()
    raise SystemExit(f"unknown workload {name}")


class StepRunner:
    """Holds the device state of one workload and runs decode steps through the library."""

    def __init__(self, w, total_steps: int, partition: int = 0, shared: bool = False):
        import torch
        import inputs
        import paged_kv_cache_284_amd as pkv
        self.torch, self.pkv, self.w = torch, pkv, w
        self.partition = partition
        self.shared = shared  # decode with pa_decode_shared_prefix
        order = inputs.free_order(w)
        self.alloc = pkv.Allocator(w.NB, w.bs, order)
        ids = pkv.run_script(self.alloc, inputs.setup_script(w))
        self.seqs = np.array([ids[b] for b in range(w.B)], np.int32)
        steps_len = total_steps if w.append else 0
        self.MB = (int(w.cached_lengths.max()) + steps_len + w.bs - 1) // w.bs + 1
        tables, lens = self.alloc.export(self.seqs, self.MB)
        self.lens = lens.astype(np.int32)
        pool = inputs.pool(w)
        dev = "cuda"

        def up(a, dt):
            a = np.ascontiguousarray(a)
            if dt == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)
        self.k = up(pool["k"], w.kv_dtype)
        self.v = up(pool["v"], w.kv_dtype)
        self.ks = self.vs = None
        if w.kv_dtype in ("i8", "i4"):
            self.ks = up(pool["k_scale"], "f32")
            self.vs = up(pool["v_scale"], "f32")
        del pool
        self.tables = torch.from_numpy(tables).to(dev)
        # per-step inputs, resident before timing
        n_inputs = max(total_steps, 1)
        self.q = [up(inputs.queries(w, s), w.q_dtype) for s in range(n_inputs)]
        self.new = []
        if w.append:
            for s in range(n_inputs):
                kn, vn = inputs.new_tokens(w, s)
                self.new.append((up(kn, w.kv_dtype), up(vn, w.kv_dtype)))
        max_len = int(self.lens.max()) + (total_steps if w.append else 0)
        ws = (pkv.decode_shared_prefix_workspace_size(w.B, w.Hq, w.Hkv, w.D, max_len) if shared
              else pkv.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, max_len, partition))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
        # the per-step host arrays, written by pa_step straight into pinned memory and read there
        # by the kernels: slots int64[B] | seq_lens int32[B] | table_index int32[B] | cow pairs
        # int32[B][2]; two pinned buffers used in turn
        B = w.B
        self.off = [0, 8 * B, 12 * B, 16 * B]
        nbytes = 24 * B
        self.pinned = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        self.hev = HipEvents()
        # decode timing events, recorded before / after each decode; the one before step s's
        # decode also marks the end of the launches that read pinned buffer s % 2
        self.n_ev = total_steps + 2
        self.ev_before = [self.hev.create() for _ in range(self.n_ev)]
        self.ev_after = [self.hev.create() for _ in range(self.n_ev)]
        self.ev_append = [self.hev.create() for _ in range(self.n_ev)]  # before copies + append
        self.timed = []
        self.lens_step = torch.empty(B, dtype=torch.int32, device=dev)  # written by the append
        self.step_no = 0
        self.max_len = int(self.lens.max())
        # ctypes arguments that do not change from step to step
        import ctypes as C
        self.C = C
        L = pkv.lib()
        self.L = L
        self.n_cow = C.c_int32()
        self.seqs_p = self.seqs.ctypes.data_as(C.POINTER(C.c_int32))
        self.hp = [[C.cast(pb.data_ptr() + o, C.POINTER(C.c_int64 if j == 0 else C.c_int32))
                    for j, o in enumerate(self.off)] for pb in self.pinned]
        self.raw = [[pb.data_ptr() + o for o in self.off] for pb in self.pinned]
        self.kv_code = {"f32": pkv.PA_F32, "bf16": pkv.PA_BF16, "i8": pkv.PA_I8,
                        "i4": pkv.PA_I4}[w.kv_dtype]
        self.q_code = {"f32": pkv.PA_F32, "bf16": pkv.PA_BF16}[w.q_dtype]
        self.stream = torch.cuda.current_stream().cuda_stream
        self.ks_p = self.ks.data_ptr() if self.ks is not None else None
        self.vs_p = self.vs.data_ptr() if self.vs is not None else None
        if not w.append:
            self.lens_dev = torch.from_numpy(self.lens).to(dev)

    def step(self, time_decode: bool = False):
        """One decode step through the C ABI: allocator step into pinned memory, copy-on-write
        copies (if any), fused append + table patch + length copy reading the pinned arrays,
        decode."""
        torch, pkv, w, L = self.torch, self.pkv, self.w, self.L
        s = self.step_no
        if w.append:
            i = s % 2
            if s >= 2:
                self.hev.sync(self.ev_before[s - 2])
            hp = self.hp[i]
            st = L.pa_step(self.alloc._h, self.seqs_p, w.B, hp[0], hp[1], hp[2], hp[3],
                           self.C.byref(self.n_cow))
            if st != 0:
                raise pkv.PagedKVError(st, "pa_step")
            h_slots, h_lens, h_tidx, h_pairs = self.raw[i]
            self.max_len += 1
            n_cow = self.n_cow.value
            self.hev.record(self.ev_append[s], self.stream)
            if n_cow:
                st = L.pa_copy_blocks(self.k.data_ptr(), self.v.data_ptr(), self.ks_p, self.vs_p,
                                      h_pairs, n_cow, w.Hkv, w.D, w.bs, w.NB, self.kv_code,
                                      self.stream)
                if st != 0:
                    raise pkv.PagedKVError(st, "pa_copy_blocks")
            kn, vn = self.new[s % len(self.new)]
            lens_d = self.lens_step.data_ptr()
            st = L.pa_append_step(kn.data_ptr(), vn.data_ptr(), h_slots, h_tidx, h_lens, lens_d,
                                  self.k.data_ptr(), self.v.data_ptr(), self.tables.data_ptr(),
                                  self.MB, w.B, w.Hkv, w.D, w.bs, w.NB, self.kv_code, self.stream)
            if st != 0:
                raise pkv.PagedKVError(st, "pa_append_step")
            self.lens += 1
        else:
            lens_d = self.lens_dev.data_ptr()
        self.hev.record(self.ev_before[s], self.stream)
        self.lens_d = lens_d
        self.decode(self.q[s % len(self.q)])
        self.hev.record(self.ev_after[s], self.stream)
        if time_decode:
            self.timed.append((s, self.lens.copy(), n_cow if w.append else 0))
        self.step_no += 1

    def decode(self, q):
        """pa_decode (or pa_decode_shared_prefix) over the current cache state (no allocator or
        cache change)."""
        w = self.w
        if self.shared:
            st = self.L.pa_decode_shared_prefix(
                self.out.data_ptr(), q.data_ptr(), self.q_code, self.k.data_ptr(),
                self.v.data_ptr(), self.kv_code, self.ks_p, self.vs_p, self.tables.data_ptr(),
                self.MB, self.lens_d, self.max_len, w.B, w.Hq, w.Hkv, w.D, w.bs, w.NB, w.scale,
                self.ws.data_ptr(), self.ws.numel(), self.stream)
            if st != 0:
                raise self.pkv.PagedKVError(st, "pa_decode_shared_prefix")
            return
        st = self.L.pa_decode(self.out.data_ptr(), q.data_ptr(), self.q_code, self.k.data_ptr(),
                              self.v.data_ptr(), self.kv_code, self.ks_p, self.vs_p,
                              self.tables.data_ptr(), self.MB, self.lens_d, self.max_len, w.B,
                              w.Hq, w.Hkv, w.D, w.bs, w.NB, w.scale, self.partition,
                              self.ws.data_ptr(), self.ws.numel(), self.stream)
        if st != 0:
            raise self.pkv.PagedKVError(st, "pa_decode")

    def decode_ms(self):
        """(ms, lengths) of every timed decode launch (after the stream has drained)."""
        return [(self.hev.elapsed_ms(self.ev_before[s], self.ev_after[s]), lens)
                for s, lens, _ in self.timed]

    def append_ms(self):
        """(ms, copy-on-write pairs) of the copies + append of every timed step."""
        if not self.w.append:
            return []
        return [(self.hev.elapsed_ms(self.ev_append[s], self.ev_before[s]), n_cow)
                for s, _, n_cow in self.timed]

    def cold_decode_ms(self, reps: int, scrub_bytes: int = 1 << 30):
        """Decode launches timed alone, each after a read of scrub_bytes of other memory (4x the
        256 MB last-level cache), as the previous layer's attention would leave the caches: no
        K/V line or translation cached, and no dirty line left to write back.  Events bracket
        the decode only."""
        torch = self.torch
        scrub = torch.ones(scrub_bytes // 4, dtype=torch.float32, device="cuda")
        total = torch.empty((), dtype=torch.float32, device="cuda")
        ev = [(self.hev.create(), self.hev.create()) for _ in range(reps)]
        q = self.q[(self.step_no - 1) % len(self.q)]
        for a, b in ev:
            torch.sum(scrub, dim=0, out=total)
            self.hev.record(a, self.stream)
            self.decode(q)
            self.hev.record(b, self.stream)
        torch.cuda.synchronize()
        del scrub, total
        return [self.hev.elapsed_ms(a, b) for a, b in ev]


def prefill_flops(w, lens, chunks) -> int:
    """Algorithmic flops of a chunked prefill: for every query (position p) and query head,
    2 D per key for the scores and 2 D per key for P.V over keys 0..p."""
    total_keys = 0
    for L, n in zip(lens, chunks):
        L, n = int(L), int(n)
        first = L - n + 1                      # keys seen by the chunk's first query
        total_keys += n * first + n * (n - 1) // 2
    return 4 * w.D * w.Hq * total_keys


class PrefillRunner:
    """Device state of a chunked-prefill workload: the cache holds each sequence's context, the
    step rewrites the chunk's K/V (one append entry per token: pa_kv_append, or the quantising
    append for int8 / int4 caches) and runs pa_prefill."""

    def __init__(self, w, chunks):
        import torch
        import inputs
        import paged_kv_cache_284_amd as pkv
        self.torch, self.pkv, self.w = torch, pkv, w
        alloc = pkv.Allocator(w.NB, w.bs, inputs.free_order(w))
        ids = pkv.run_script(alloc, inputs.setup_script(w))
        seqs = [ids[b] for b in range(w.B)]
        self.MB = (int(w.lengths.max()) + w.bs - 1) // w.bs + 1
        tables, lens = alloc.export(seqs, self.MB)
        self.lens_h = lens.astype(np.int32)
        self.chunks = np.asarray(chunks, np.int64)
        cu = np.concatenate([[0], np.cumsum(self.chunks)]).astype(np.int32)
        self.T = int(cu[-1])
        # slots of the chunk tokens: the last n_b positions of each sequence
        slots = []
        ks, vs = [], []
        for b in range(w.B):
            L, n = int(lens[b]), int(self.chunks[b])
            for p in range(L - n, L):
                slots.append(int(tables[b][p // w.bs]) * w.bs + p % w.bs)
            # quantised caches take bf16 tokens through the quantising append
            kn, vn = inputs.token_kv(w.cid, b, n, w.Hkv, w.D,
                                     "bf16" if w.kv_dtype in ("i8", "i4") else w.kv_dtype)
            ks.append(kn)
            vs.append(vn)
        pool = inputs.pool(w)

        def up(a):
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        self.ks = self.vs = None
        if w.kv_dtype in ("i8", "i4"):
            self.k = torch.from_numpy(np.ascontiguousarray(pool["k"])).cuda()
            self.v = torch.from_numpy(np.ascontiguousarray(pool["v"])).cuda()
            self.ks = torch.from_numpy(pool["k_scale"]).cuda()
            self.vs = torch.from_numpy(pool["v_scale"]).cuda()
        else:
            self.k, self.v = up(pool["k"]), up(pool["v"])
        del pool
        self.k_new, self.v_new = up(np.concatenate(ks)), up(np.concatenate(vs))
        self.slots = torch.tensor(slots, dtype=torch.int64, device="cuda")
        self.tables = torch.from_numpy(tables).cuda()
        self.lens = torch.from_numpy(self.lens_h).cuda()
        self.cu = torch.from_numpy(cu).cuda()
        self.q = up(inputs.chunk_queries(w, self.T))
        self.out = torch.empty((self.T, w.Hq, w.D), dtype=torch.float32, device="cuda")
        self.hev = HipEvents()
        self.stream = torch.cuda.current_stream().cuda_stream
        self.events = []

    def step(self, time_it: bool = False):
        pkv, w = self.pkv, self.w
        if w.kv_dtype == "i8":
            pkv.kv_append_int8(self.k_new, self.v_new, self.slots, self.k, self.v, self.ks, self.vs)
        elif w.kv_dtype == "i4":
            pkv.kv_append_int4(self.k_new, self.v_new, self.slots, self.k, self.v, self.ks, self.vs)
        else:
            pkv.kv_append(self.k_new, self.v_new, self.slots, self.k, self.v)
        e0 = e1 = None
        if time_it:
            e0, e1 = self.hev.create(), self.hev.create()
            self.hev.record(e0, self.stream)
        pkv.prefill(self.q, self.k, self.v, self.tables, self.lens, self.cu,
                    int(self.lens_h.max()), w.scale, k_scale=self.ks, v_scale=self.vs,
                    out=self.out)
        if time_it:
            self.hev.record(e1, self.stream)
            self.events.append((e0, e1))

    def prefill_ms(self):
        return [self.hev.elapsed_ms(a, b) for a, b in self.events]


PREFILL_KV = {"prefill_llama8b": "bf16", "prefill_llama8b_i8": "i8", "prefill_llama8b_i4": "i4"}


def prefill_workload(name: str = "prefill_llama8b"):
    """Llama-3.1-8B heads, B 8, contexts U[2048, 4096] ending in a 512-token chunk each; the
    _i8 / _i4 variants keep the cache as int8 or packed int4 codes with per-block scales."""
    import inputs
    w = inputs.llama8b_decode(B=8, lo=2048, hi=4096, cid=72, name=name)
    w.append = False
    w.kv_dtype = PREFILL_KV[name]
    return w, inputs.chunk_sizes(w, 512, 512)


def cpu_baseline_prefill(name: str, min_seconds: float = 10.0) -> dict:
    """The fp64 oracle on sampled (query row, head) pairs of the prefill workload, one thread,
    scaled to query tokens/s (a token is Hq row-heads)."""
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    code = f"""
import sys, time, json, numpy as np
sys.path.insert(0, {ROOT!r})
import inputs
from oracle.allocator import PyAllocator, run_script
from oracle.prefill import prefill_paged
from bench import prefill_workload
w, chunks = prefill_workload({name!r})
a = PyAllocator(w.NB, w.bs, inputs.free_order(w))
ids = run_script(a, inputs.setup_script(w))
seqs = [ids[b] for b in range(w.B)]
tables, lens = a.export(seqs, max(len(a.table(s)) for s in seqs))
pool = inputs.pool(w)
cu = np.concatenate([[0], np.cumsum(chunks)])
T = int(cu[-1])
q = inputs.chunk_queries(w, T)
rng = np.random.default_rng(0)
done, t0 = 0, time.perf_counter()
while True:
    b = int(rng.integers(0, w.B))
    g = int(rng.integers(0, w.Hkv))
    rows = [(int(cu[b]) + int(i), h) for i in rng.integers(0, int(chunks[b]), 32)
            for h in range(g * w.G, (g + 1) * w.G)]
    prefill_paged(q[cu[b]:cu[b + 1]], w.q_dtype, pool["k"], pool["v"], w.kv_dtype, [tables[b]],
                  [lens[b]], [0, int(chunks[b])], w.bs, w.scale, pool.get("k_scale"),
                  pool.get("v_scale"), rows=[(r - int(cu[b]), h) for r, h in rows])
    done += len(rows)
    el = time.perf_counter() - t0
    if el >= {min_seconds}:
        break
print(json.dumps({{"rowheads": done, "seconds": el}}))
"""
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=ROOT)
    if r.returncode != 0:
        raise RuntimeError(r.stderr[-2000:])
    d = json.loads(r.stdout.strip().splitlines()[-1])
    w, _ = prefill_workload(name)
    return {"value": round(d["rowheads"] / w.Hq / d["seconds"], 2), "unit": "tokens/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{d['rowheads']} sampled (query row, head) outputs of the workload "
                      f"(32 rows x the G heads of one KV head per draw, fp64 numpy, 1 thread) "
                      f"in {d['seconds']:.1f} s"}


def run_prefill(args):
    import torch
    w, chunks = prefill_workload(args.workload)
    runner = PrefillRunner(w, chunks)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        runner.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        runner.step(time_it=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = runner.prefill_ms()
    mean_ms = float(np.mean(ms))
    flops = prefill_flops(w, runner.lens_h, chunks)
    tflops = flops / (mean_ms * 1e-3) / 1e12
    rec = {
        "metric": "paged chunked-prefill attn: query tokens/s + achieved MFMA TFLOP/s",
        "value": round(runner.T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic (seeded N(0,1) K/V/q, shapes of the workload; no weights)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D,
                   "block_size": w.bs, "kv_dtype": w.kv_dtype,
                   "chunk_tokens": [int(c) for c in chunks],
                   "context_tokens": [int(x) for x in runner.lens_h]},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "prefill_ms_mean": round(mean_ms, 5),
        "prefill_algorithmic_flops": flops,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_prefill(args.workload, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


# host link of an MI355X: PCIe 5.0 x16, 32 GT/s x 16 lanes x 128/130 encoding, per direction
PEAK_HOST_LINK_GBPS = 63.0
SWAP_WORKLOAD = "swap_llama8b"


def run_swap(args):
    """Preemption by swapping on the headline layer's pool (bf16, 8 KV heads, D 128, 16-token
    blocks): the blocks of 8 of its 64 sequences (seeded pick, lengths U[512, 4096]) copied to a
    pinned host swap pool with one pa_swap_blocks launch (swap-out), then back into other
    device blocks (swap-in).  Each timed step is one swap-out and one swap-in, timed apart with
    HIP events on the launch stream; the rate is the blocks' K and V bytes over the launch time,
    against the host link's per-direction peak."""
    import torch
    import paged_kv_cache_284_amd as pkv
    w = build_workload("llama8b_decode", 1)
    rng = np.random.default_rng(2024)
    picked = np.sort(rng.choice(w.B, 8, replace=False))
    nblk = int(sum((int(w.lengths[b]) + w.bs - 1) // w.bs for b in picked))
    NB = int(w.NB)
    dev = torch.device("cuda")
    k = torch.randn((NB, w.Hkv, w.bs, w.D), dtype=torch.bfloat16, device=dev)
    v = torch.randn((NB, w.Hkv, w.D, w.bs), dtype=torch.bfloat16, device=dev)
    hk = torch.empty((nblk, w.Hkv, w.bs, w.D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty((nblk, w.Hkv, w.D, w.bs), dtype=torch.bfloat16, pin_memory=True)
    blocks = rng.permutation(NB)
    out_src, in_dst = blocks[:nblk], blocks[nblk:2 * nblk]
    host = np.arange(nblk)
    pairs_out = torch.from_numpy(np.stack([out_src, host], 1).astype(np.int32)).to(dev)
    pairs_in = torch.from_numpy(np.stack([host, in_dst], 1).astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream()
    ev = HipEvents()
    sid = stream.cuda_stream
    for _ in range(args.warmup):
        pkv.swap_blocks(k, v, hk, hv, pairs_out, stream=stream)
        pkv.swap_blocks(hk, hv, k, v, pairs_in, stream=stream)
    torch.cuda.synchronize()
    marks = [ev.create() for _ in range(3 * args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev.record(marks[3 * i], sid)
        pkv.swap_blocks(k, v, hk, hv, pairs_out, stream=stream)
        ev.record(marks[3 * i + 1], sid)
        pkv.swap_blocks(hk, hv, k, v, pairs_in, stream=stream)
        ev.record(marks[3 * i + 2], sid)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    out_ms = [ev.elapsed_ms(marks[3 * i], marks[3 * i + 1]) for i in range(args.steps)]
    in_ms = [ev.elapsed_ms(marks[3 * i + 1], marks[3 * i + 2]) for i in range(args.steps)]
    for e in marks:
        ev.hip.hipEventDestroy(e)
    nbytes = nblk * 2 * w.Hkv * w.bs * w.D * 2
    out_gbps = nbytes / (float(np.mean(out_ms)) * 1e-3) / 1e9
    in_gbps = nbytes / (float(np.mean(in_ms)) * 1e-3) / 1e9
    achieved = 2 * nbytes / ((float(np.mean(out_ms)) + float(np.mean(in_ms))) * 1e-3) / 1e9
    rec = {
        "metric": "pa_swap_blocks: KV bytes moved per second between HBM and a pinned host pool",
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V in the headline layer's pool shape; no weights)",
        "config": {"workload": SWAP_WORKLOAD, "Hkv": w.Hkv, "head_dim": w.D, "block_size": w.bs,
                   "kv_dtype": "bf16", "pool_blocks": NB, "sequences": [int(b) for b in picked],
                   "blocks_per_swap": nblk, "bytes_per_swap": nbytes},
        "roofline": {"bound": "host link", "achieved": round(achieved, 2),
                     "peak": PEAK_HOST_LINK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HOST_LINK_GBPS, 4), "traffic": None},
        "swap_out_ms_mean": round(float(np.mean(out_ms)), 5),
        "swap_in_ms_mean": round(float(np.mean(in_ms)), 5),
        "swap_out_gbps": round(out_gbps, 2),
        "swap_in_gbps": round(in_gbps, 2),
    }
    print(json.dumps(rec), flush=True)


PREFIX_WORKLOAD = "prefix_cache_host"


def run_prefix_cache(args):
    """Automatic prefix caching on the host allocator (no GPU work): a 3,000-token prompt is
    cached once (created, its slots reserved, its full blocks published), then each request
    shares it and adds 64 tokens of its own: pa_seq_create_prefix hashes the prompt's blocks
    (chained FNV-1a over the parent hash and 16 token ids) and finds 187 of them cached (2,992
    tokens), and pa_seq_reserve takes slots for the other 72.  Requests are released after each
    round of 64, so their private blocks become evictable (and are evicted, oldest first, once
    the free list is empty).  Timed: `steps` rounds of create + reserve + release, called through
    the C ABI with every argument prepared beforehand (Python's own marshalling, several
    microseconds per call, would otherwise dominate)."""
    import ctypes as C
    import paged_kv_cache_284_amd as pkv
    L = pkv.lib()
    rng = np.random.default_rng(3000)
    prompt = rng.integers(0, 128000, 3000).astype(np.int32)
    rounds = args.warmup + args.steps
    reqs = [[np.concatenate([prompt, rng.integers(0, 128000, 64).astype(np.int32)])
             for _ in range(64)] for _ in range(rounds)]
    ptrs = [[r.ctypes.data_as(C.POINTER(C.c_int32)) for r in rr] for rr in reqs]
    al = pkv.Allocator(4096, 16)
    s0, c0 = al.create_prefix(np.concatenate([prompt, np.ones(1, np.int32)]))
    al.reserve(s0, len(prompt) + 1 - c0)
    slots = np.zeros(128, np.int64)
    pairs = np.zeros((128, 2), np.int32)
    p_slots = slots.ctypes.data_as(C.POINTER(C.c_int64))
    p_pairs = pairs.ctypes.data_as(C.POINTER(C.c_int32))
    seq, cached, ncow = C.c_int32(), C.c_int32(), C.c_int32()
    r_seq, r_cached, r_ncow = C.byref(seq), C.byref(cached), C.byref(ncow)
    n_req = len(prompt) + 64
    h = al._h

    def round_(k):
        live, tot = [], 0
        for p in ptrs[k]:
            if L.pa_seq_create_prefix(h, p, n_req, 0, r_seq, r_cached) != 0:
                raise RuntimeError("pa_seq_create_prefix failed")
            if L.pa_seq_reserve(h, seq.value, n_req - cached.value, p_slots, p_pairs,
                                r_ncow) != 0:
                raise RuntimeError("pa_seq_reserve failed")
            live.append(seq.value)
            tot += cached.value
        for s_ in live:
            if L.pa_seq_free(h, s_) != 0:
                raise RuntimeError("pa_seq_free failed")
        return tot

    for k in range(args.warmup):
        round_(k)
    t0 = time.perf_counter()
    tot = 0
    for k in range(args.warmup, rounds):
        tot += round_(k)
    elapsed = time.perf_counter() - t0
    n = 64 * args.steps
    rec = {
        "metric": "automatic prefix caching: requests created per second on the host allocator",
        "value": round(n / elapsed, 1),
        "unit": "requests/s",
        "n_gpus": 0,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32 token ids, uint64 hashes",
        "data": "synthetic (seeded token ids; a 3,000-token shared prompt, 64 private tokens per "
                "request)",
        "config": {"workload": PREFIX_WORKLOAD, "block_size": 16, "pool_blocks": 4096,
                   "prompt_tokens": len(prompt), "private_tokens": 64,
                   "requests_per_step": 64},
        "us_per_request": round(elapsed / n * 1e6, 2),
        "cached_tokens_per_request": tot // n,
        "token_ids_hashed_per_s": round(n_req * n / elapsed, 1),
        "host": cpu_model(),
    }
    al.close()
    print(json.dumps(rec), flush=True)


def host_threads() -> int:
    """Threads this process may use: the CPU affinity, capped by OMP_NUM_THREADS when set."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(env)) if env.isdigit() and int(env) > 0 else n


def cpu_baseline(name: str, min_seconds: float = 10.0, workers: int = 1) -> dict:
    """Time the fp64 oracle on decode steps of the same workload on the host cores, in a child
    process with one BLAS thread per process (input generation excluded).  With workers > 1 the
    child forks that many processes after the set-up (sharing its arrays), each repeating the
    decode of its own share of the sequences (b = worker mod workers), and the rates add up."""
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    code = f"""
import sys, time, json, numpy as np
import multiprocessing as mp
sys.path.insert(0, {ROOT!r})
import inputs
from oracle import attention
from oracle.allocator import PyAllocator, run_script
from bench import build_workload
w = build_workload({name!r}, 1)
a = PyAllocator(w.NB, w.bs, inputs.free_order(w))
ids = run_script(a, inputs.setup_script(w))
seqs = [ids[b] for b in range(w.B)]
if w.append:
    a.step(seqs)
tables, lens = a.export(seqs, max(len(a.table(s)) for s in seqs))
tables, lens = np.asarray(tables), np.asarray(lens)
pool = inputs.pool(w)
q = inputs.queries(w, 0)
N = {workers}
def work(i):
    idx = np.arange(i, w.B, N)
    if len(idx) == 0:
        return (0, 0, 1.0)
    reps, t0 = 0, time.perf_counter()
    while True:
        attention.decode_paged(q[idx], w.q_dtype, pool["k"], pool["v"], w.kv_dtype, tables[idx],
                               lens[idx], w.bs, w.scale, pool.get("k_scale"), pool.get("v_scale"))
        reps += 1
        el = time.perf_counter() - t0
        if el >= {min_seconds}:
            return (len(idx), reps, el)
if N == 1:
    res = [work(0)]
else:
    with mp.get_context("fork").Pool(N) as p:
        res = p.map(work, range(N))
print(json.dumps({{"res": res, "B": w.B}}))
"""
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=ROOT)
    if r.returncode != 0:
        return {"value": None, "unit": "tokens/s", "cores": workers, "kind": "oracle",
                "sample": f"failed: {r.stderr[-300:]}"}
    d = json.loads(r.stdout.strip().splitlines()[-1])
    tps = sum(n * reps / el for n, reps, el in d["res"] if n)
    steps = sum(n * reps for n, reps, _ in d["res"]) / d["B"]
    secs = max(el for _, _, el in d["res"])
    what = ("1 process" if workers == 1 else
            f"{workers} processes of one thread, each over every {workers}th sequence")
    return {"value": round(tps, 3), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{steps:.1f} full decode step(s) of the workload (B={d['B']}, all heads, "
                      f"fp64 numpy, {what}) in {secs:.1f} s"}


def stream_copy_gbps(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Device-to-device copy rate (bytes read + written per second) of the runtime's copy, for
    context beside the decode rate."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    hev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    a, b = hev.create(), hev.create()
    hev.record(a, stream)
    for _ in range(reps):
        dst.copy_(src)
    hev.record(b, stream)
    torch.cuda.synchronize()
    ms = hev.elapsed_ms(a, b)
    del src, dst
    return round(2 * nbytes * reps / (ms * 1e-3) / 1e9, 1)


def traffic_from_profiles(kernel_src_hash: str):
    """HBM bytes per decode launch from the committed counter summary, when it was taken on the
    current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_sources_sha256") != kernel_src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


DECODE_SOURCES = ("decode_mfma.hip", "device_load.h", "internal.h", "quant_f16.h")
# the balanced bf16 decode kernel of the Llama-3.1-8B-shaped batch (G = 4, D = 128)
DECODE_KERNEL = "decode_mfma_kernel<4, 128, 1, 0>"
TRAFFIC_WORKLOAD = "llama8b_decode"


def kernel_sources_hash() -> str:
    """sha256 over the code of the sources the decode kernel is built from: each line with its
    // comment and surrounding blanks removed, empty lines dropped (comment edits keep it)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_284_amd", "csrc")
    for f in DECODE_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = [ln.split("//", 1)[0].strip() for ln in fh]
        h.update(f.encode() + "\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()


def summarize_counters(d: str, copy_mib: int = 512) -> dict:
    """profiles/decode_traffic.json from the four rocprofv3 --pmc runs listed in it (FETCH_SIZE
    and WRITE_SIZE, in KiB per dispatch, on the decode bench and on a plain copy of copy_mib
    MiB): the decode kernel's counters scaled by what the same counters read for the copy's
    known bytes."""
    import csv

    def rows(sub, prefix):
        with open(os.path.join(d, sub, f"{prefix}_counter_collection.csv")) as f:
            return list(csv.DictReader(f))

    def mean(vals):
        return sum(vals) / len(vals)

    dec_f = [float(r["Counter_Value"]) for r in rows("pmc_FETCH_SIZE", "dec")
             if DECODE_KERNEL in r["Kernel_Name"]]
    dec_w = [float(r["Counter_Value"]) for r in rows("pmc_WRITE_SIZE", "dec")
             if DECODE_KERNEL in r["Kernel_Name"]]
    if not dec_f or not dec_w:
        raise SystemExit(f"no {DECODE_KERNEL} dispatch in the counter runs under {d}")
    # the device-to-device copy torch issues for Tensor.copy_ (the fill before it is skipped)
    big = lambda rs: [float(r["Counter_Value"]) for r in rs  # noqa: E731
                      if "copyBuffer" in r["Kernel_Name"]]
    cp_f = big(rows("pmc_copy_FETCH_SIZE", "cp"))
    cp_w = big(rows("pmc_copy_WRITE_SIZE", "cp"))
    known_kib = copy_mib * 1024
    fs, ws = known_kib / mean(cp_f), known_kib / mean(cp_w)
    out = {
        "kernel": "decode_mfma_kernel<4, 128, balanced, bf16>",
        "workload": "llama8b_decode (B=64, 32/8 heads, D=128, bf16, L ~ U[512,4096])",
        "fetch_kib_per_dispatch": round(mean(dec_f), 1),
        "write_kib_per_dispatch": round(mean(dec_w), 1),
        "copy_reference_mib": copy_mib,
        "copy_fetch_kib_per_dispatch": round(mean(cp_f), 1),
        "copy_write_kib_per_dispatch": round(mean(cp_w), 1),
        "fetch_scale": round(fs, 4),
        "write_scale": round(ws, 4),
        "hbm_bytes_per_launch": int((mean(dec_f) * fs + mean(dec_w) * ws) * 1024),
        "kernel_sources_sha256": kernel_sources_hash(),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d prof_out/pmc_FETCH_SIZE -o dec -- "
            "python3 -u bench.py --steps 3 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-configs",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d prof_out/pmc_WRITE_SIZE -o dec -- "
            "python3 -u bench.py --steps 3 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-configs",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d prof_out/pmc_copy_FETCH_SIZE -o cp "
            f"-- python3 -u bench.py --copy-reference {copy_mib}",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d prof_out/pmc_copy_WRITE_SIZE -o cp "
            f"-- python3 -u bench.py --copy-reference {copy_mib}",
            "python3 bench.py --summarize-counters prof_out",
        ],
    }
    return out


def release_device_memory():
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def settle(ms: float, runner) -> float:
    """Before timing, decode the workload's first-step state for `ms` of wall time with the
    fixed-partition schedule at 8192 tokens (pa_decode with partition_tokens 8192: one
    workgroup per sequence and KV head, no merge launch).  The calls read the same pool pages
    as the timed decode and change no state; without them the first timed steps ran about 1%
    slower.  They use other kernel instances than the balanced schedule, so a trace keeps the
    timed kernels' rows apart from them."""
    import torch
    w = runner.w
    if w.q_dtype != "bf16" or w.kv_dtype not in ("bf16", "i8", "i4"):
        return 0.0  # the portable kernel serves these: no separate instance to settle with
    runner.lens_d = runner.lens_dev.data_ptr() if not w.append else runner.lens_step.data_ptr()
    if w.append:
        runner.lens_step.copy_(torch.from_numpy(runner.lens))
    pkv = runner.pkv
    ws = torch.empty(max(pkv.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, runner.max_len, 8192),
                         1), dtype=torch.uint8, device="cuda")
    q = runner.q[0]
    t_end = time.perf_counter() + ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(20):
            st = runner.L.pa_decode(
                runner.out.data_ptr(), q.data_ptr(), runner.q_code, runner.k.data_ptr(),
                runner.v.data_ptr(), runner.kv_code, runner.ks_p, runner.vs_p,
                runner.tables.data_ptr(), runner.MB, runner.lens_d, runner.max_len, w.B, w.Hq,
                w.Hkv, w.D, w.bs, w.NB, w.scale, 8192, ws.data_ptr(), ws.numel(), runner.stream)
            if st != 0:
                raise pkv.PagedKVError(st, "pa_decode")
        torch.cuda.synchronize()
    del ws
    return ms


def measure_decode(name: str, steps: int, warmup: int, cold_reps: int, partition: int = 0,
                   shared: bool = False, settle_ms: float = 0.0):
    """Run warmup + steps decode steps of a workload through the library (each step: allocator
    step, copy-on-write copies, append, decode, for workloads that append) and time them.
    shared: decode with pa_decode_shared_prefix.  settle_ms: before the warm-up steps, repeat
    untimed decode calls on the first step's state (they change no state) for that long, so
    that the GPU's clocks reach the level they hold under sustained load."""
    import torch
    total = warmup + steps
    w = build_workload(name, total)
    runner = StepRunner(w, total, partition, shared)
    settled = settle(settle_ms, runner) if settle_ms > 0 else 0.0
    if warmup == 0:
        # timing from the first step (its copy-on-write copies included): one decode call
        # beforehand, which changes no state, loads the kernels' code outside the timed steps
        runner.lens_d = runner.lens_dev.data_ptr() if not w.append else runner.lens_step.data_ptr()
        if w.append:
            runner.lens_step.copy_(torch.from_numpy(runner.lens))
        runner.decode(runner.q[0])
    torch.cuda.synchronize()
    for _ in range(warmup):
        runner.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        runner.step(time_decode=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed = runner.decode_ms()
    ms = [t for t, _ in timed]
    # the tables after the last step serve every timed step: a copy-on-write only ever replaces
    # a shared block by a private copy, and blocks a later step adds hold no token of an earlier
    tables_now, _ = runner.alloc.export(runner.seqs, runner.MB)
    logical = [algorithmic_bytes(w, lens) for _, lens in timed]
    byts = [algorithmic_bytes(w, lens, tables_now) for _, lens in timed]
    mean_ms = float(np.mean(ms))
    out = {"w": w, "elapsed": elapsed, "ms": ms, "mean_ms": mean_ms, "bytes": byts,
           "logical": logical, "achieved": float(np.mean(byts)) / (mean_ms * 1e-3) / 1e9,
           "append": runner.append_ms(), "settled_ms": settled,
           "cold": runner.cold_decode_ms(cold_reps) if cold_reps else []}
    del runner
    return out


# The decode configurations of the workload list, measured after the headline and reported
# beside it.  Workloads that append run from their first step (warm-up 0), so that the shared-
# prefix batch's copy-on-write step is inside the timed steps.
CONFIG_WORKLOADS = ("tiny_fp32", "llama8b_decode", "long_context", "shared_prefix_batch",
                    "int8_mha", "int4_mha", "llama8b_decode_tp8")
CONFIG_STEPS = {"tiny_fp32": (0, 10), "llama8b_decode": (2, 10), "long_context": (2, 8),
                "shared_prefix_batch": (0, 12), "int8_mha": (3, 12), "int4_mha": (3, 12),
                "llama8b_decode_tp8": (2, 10)}


# Workloads whose sequences share prefixes: their record is the shared-prefix decode's, with
# pa_decode's time on the same steps beside it.
SHARED_PREFIX_WORKLOADS = ("shared_prefix_batch",)


def config_record(name: str) -> dict:
    """One configuration's decode figures: HIP-event time of each decode call (all its
    kernels), unique and logical algorithmic bytes, rate and fraction of the HBM peak (the tiny
    batch is latency-bound: time only), the decode after a 1 GiB read of other memory, and the
    append."""
    warmup, steps = CONFIG_STEPS[name]
    shared = name in SHARED_PREFIX_WORKLOADS
    plain = None
    if shared:
        p = measure_decode(name, steps, warmup, 0)
        plain = (float(np.median(p["ms"])), p["achieved"])
        p = None
        release_device_memory()
    m = measure_decode(name, steps, warmup, 5, shared=shared)
    w = m["w"]
    med = float(np.median(m["ms"]))
    ub, lb = float(np.mean(m["bytes"])), float(np.mean(m["logical"]))
    r = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D,
         "kv_dtype": w.kv_dtype, "warmup": warmup, "steps": steps,
         "decode": "pa_decode_shared_prefix" if shared else "pa_decode",
         "decode_us_median": round(med * 1e3, 2), "decode_us_mean": round(m["mean_ms"] * 1e3, 2),
         "unique_bytes": int(ub), "logical_bytes": int(lb)}
    if plain is not None:
        r["pa_decode_us_median"] = round(plain[0] * 1e3, 2)
        r["pa_decode_frac"] = round(plain[1] / PEAK_HBM_GBPS, 4)
    if w.name != "tiny_fp32":
        r["unique_gbps"] = round(m["achieved"], 1)
        r["logical_gbps"] = round(lb / (m["mean_ms"] * 1e-3) / 1e9, 1)
        r["frac"] = round(m["achieved"] / PEAK_HBM_GBPS, 4)
        r["tokens_per_s"] = round(w.B / (m["mean_ms"] * 1e-3), 1)
    if m["cold"]:
        r["cold_us_median"] = round(float(np.median(m["cold"])) * 1e3, 2)
    if m["append"]:
        r["append_us_mean"] = round(float(np.mean([t for t, _ in m["append"]])) * 1e3, 2)
        r["append_us_first_step"] = round(m["append"][0][0] * 1e3, 2)
        r["cow_pairs_first_step"] = int(m["append"][0][1])
        r["cow_pairs_timed"] = int(sum(n for _, n in m["append"]))
    m = None
    release_device_memory()
    return r


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed decode calls on the first step's state for this long before "
                         "the warm-up steps (the GPU at its sustained state when timing starts)")
    ap.add_argument("--workload", default="llama8b_decode")
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--shared-prefix", action="store_true",
                    help="decode with pa_decode_shared_prefix")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration records after the headline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="decode launches timed alone after a 1 GiB read of other memory "
                         "(0: skip)")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters against known bytes) and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write profiles/decode_traffic.json from the rocprofv3 --pmc runs under "
                         "DIR (no GPU needed) and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        out = summarize_counters(args.summarize_counters)
        with open(os.path.join(ROOT, "profiles", "decode_traffic.json"), "w") as f:
            json.dump(out, f, indent=1)
        print(json.dumps(out))
        return
    if args.workload == PREFIX_WORKLOAD:
        run_prefix_cache(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path shards by sequence or KV head with no "
              "exchange, and it runs and reports a single MI355X only.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    if args.copy_reference:
        n = args.copy_reference << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_reference_bytes_read": n, "copy_reference_bytes_written": n,
                          "launches": 5}))
        return

    import paged_kv_cache_284_amd as pkv
    pkv.lib()
    if args.workload == SWAP_WORKLOAD:
        run_swap(args)
        return
    if args.workload.startswith("prefill"):
        run_prefill(args)
        return

    m = measure_decode(args.workload, args.steps, args.warmup, args.cold_reps, args.partition,
                       args.shared_prefix, args.settle_ms)
    w = m["w"]
    # the committed counters cover the headline batch only
    traffic = (traffic_from_profiles(kernel_sources_hash())
               if args.workload == TRAFFIC_WORKLOAD else None)
    rec = {
        "metric": METRIC,
        "value": round(w.B * args.steps / m["elapsed"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": m["settled_ms"],
        "ms_per_step": round(m["elapsed"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic (seeded N(0,1) K/V/q, shapes of the workload; no weights)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D,
                   "block_size": w.bs, "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype,
                   "context_tokens_first_step": int(w.lengths.sum()), "pool_blocks": w.NB,
                   "partition_tokens": args.partition or "auto",
                   "decode": "pa_decode_shared_prefix" if args.shared_prefix else "pa_decode"},
        "roofline": {"bound": "hbm", "achieved": round(m["achieved"], 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(m["achieved"] / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
        "decode_ms_mean": round(m["mean_ms"], 5),
        "decode_ms_median": round(float(np.median(m["ms"])), 5),
        "decode_ms_p10_p90": [round(float(np.percentile(m["ms"], 10)), 5),
                              round(float(np.percentile(m["ms"], 90)), 5)],
        "decode_algorithmic_bytes_mean": int(np.mean(m["bytes"])),
        "decode_logical_bytes_mean": int(np.mean(m["logical"])),
        "decode_tokens_per_s": round(w.B / (m["mean_ms"] * 1e-3), 1),
    }
    if m["append"]:
        rec["append_ms_mean"] = round(float(np.mean([t for t, _ in m["append"]])), 5)
        rec["append_cow_pairs_timed"] = int(sum(n for _, n in m["append"]))
    if m["cold"]:
        cmed = float(np.median(m["cold"]))
        rec["decode_cold_ms_median"] = round(cmed, 5)
        rec["decode_cold_gbps"] = round(float(np.mean(m["bytes"])) / (cmed * 1e-3) / 1e9, 1)
    m = None
    release_device_memory()
    rec["stream_copy_gbps"] = stream_copy_gbps()
    if not args.no_configs:
        rec["configs"] = [config_record(name) for name in CONFIG_WORKLOADS]
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
        n = host_threads()
        if n > 1:
            rec["cpu_baseline_all_cores"] = cpu_baseline(args.workload, args.cpu_seconds / 2,
                                                         workers=n)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
