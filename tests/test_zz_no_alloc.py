"""GPU: pa_decode_no_alloc (the library's fixed device scratch; nothing allocated) against
pa_decode with a caller workspace, through the C-ABI: two calls in a row, the second with a
smaller batch, for both schedules, and the rejection of a call that needs more scratch."""
import ctypes as C

import numpy as np
import pytest
import torch

import inputs
import paged_kv_cache_284_amd as pkv
from tests.gpu_cases import TOL, Case, max_err, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,partition", [("llama8b_decode", 0), ("long_context", 0),
                                            ("int8_mha", 0), ("int4_mha", 0),
                                            ("llama8b_decode", 64), ("tiny_fp32", 0)])
def test_no_alloc_matches_workspace_call(name, partition):
    w = inputs.small(name)
    case = Case(w)
    q, _, tables, lens = case.step(partition_tokens=partition)
    qd = to_device(q, w.q_dtype)
    lens_d = torch.from_numpy(lens).cuda()
    L = int(lens.max())
    for nb in (w.B, max(1, w.B // 2)):
        say(f"no-alloc {w.name} partition {partition}: {nb} of {w.B} sequences")
        want = pkv.decode(qd[:nb], case.k, case.v, case.tables[:nb], lens_d[:nb], L, w.scale,
                          case.ks, case.vs, partition_tokens=partition)
        out = torch.full((nb, w.Hq, w.D), float("nan"), dtype=torch.float32, device="cuda")
        pkv.decode_no_alloc(qd[:nb], case.k, case.v, case.tables[:nb], lens_d[:nb], L, w.scale,
                            out, case.ks, case.vs, partition_tokens=partition)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, want.cpu().numpy())
        ref = case.oracle(q[:nb], tables[:nb], lens[:nb])
        assert max_err(got, ref) <= TOL[w.kv_dtype]


def test_no_alloc_rejects_more_than_its_scratch():
    """Fixed 64-token partitions over 256 sequences of 64 heads up to 4096 tokens need ~545 MB
    of partial states: the call returns PA_ERR_TOO_LARGE and writes nothing."""
    B, Hq, Hkv, D, NB, max_len = 256, 64, 8, 128, 8, 4096
    k = torch.zeros((NB, Hkv, 16, D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((NB, Hkv, D, 16), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros((B, max_len // 16), dtype=torch.int32, device="cuda")
    lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), 7.0, dtype=torch.float32, device="cuda")
    say("no-alloc: a call beyond the scratch")
    st = pkv.lib().pa_decode_no_alloc(out.data_ptr(), q.data_ptr(), pkv.PA_BF16, k.data_ptr(),
                                      v.data_ptr(), pkv.PA_BF16, None, None, tables.data_ptr(),
                                      tables.shape[1], lens.data_ptr(), max_len, B, Hq, Hkv, D,
                                      16, NB, 0.125, 64, C.c_void_p(0))
    torch.cuda.synchronize()
    assert st == pkv.PA_ERR_TOO_LARGE
    assert bool(torch.all(out == 7.0))
