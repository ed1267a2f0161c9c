"""gpuos_eager_submit_static (no allocation; split partials and counters in
the library's static device array) against gpuos_eager_submit with a caller
workspace, through the C ABI.  Both run the same op bodies with the same
split structure, so their outputs must agree bit for bit.  Two calls in a
row, the second smaller than the first: the shared array keeps the first
call's contents, so the second shows that nothing left behind leaks into
its results."""
import numpy as np
import pytest

import workloads as W
from gpu_harness import say
from oracle_util import bf16, rec
from persistent_micro_dispatch_amd import gpuos as G
from workloads.gpu import DevicePool, to_descs

pytestmark = pytest.mark.gpu


def _case(seed, B, H, C, lens, K, N, n_add):
    """Attention (split over keys), vector-matrix product (split over rows)
    and an add: arrays and records; the last three buffers are outputs."""
    rng = np.random.default_rng(seed)
    D = 128
    q = bf16(rng.standard_normal(B * H * D))
    Kc = bf16(rng.standard_normal(B * H * C * D))
    Vc = bf16(rng.standard_normal(B * H * C * D))
    x = bf16(rng.standard_normal(K))
    Wm = bf16(0.02 * rng.standard_normal(K * N))
    a = rng.standard_normal(n_add).astype(np.float32)
    b = rng.standard_normal(n_add).astype(np.float32)
    arrays = [q, Kc, Vc, x, Wm, a, b, np.zeros(B * H * D, np.float32), np.zeros(N, np.uint16),
              np.zeros(n_add, np.float32)]
    recs = np.concatenate([
        rec(W.OP_SDPA, dtype=W.BF16, out_dtype=W.F32, size=B, dim=(H, D, C, H), lens=lens,
            a=0, aux0=1, aux1=2, out=7),
        rec(W.OP_GEMV, dtype=W.BF16, out_dtype=W.BF16, dim=(K, N), a=3, b=4, out=8),
        rec(W.OP_ADD, size=n_add, a=5, b=6, out=9),
    ])
    return arrays, recs


def _run(entry, arrays, recs):
    import torch
    pool = DevicePool(arrays)
    descs = to_descs(recs, pool.ptrs)
    st = torch.cuda.Stream()
    if entry == "static":
        rc = G.gpuos_eager_submit_static(descs, st.cuda_stream)
    else:
        nb = G.gpuos_eager_scratch_bytes(descs)
        scratch = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        torch.cuda.current_stream().synchronize()
        rc = G.gpuos_eager_submit(descs, st.cuda_stream, scratch.data_ptr(), nb)
    assert rc == 0, G.ERR_NAMES.get(rc)
    st.synchronize()
    return [pool.download(i) for i in range(len(arrays) - 3, len(arrays))]


def test_static_scratch_matches_the_workspace_entry_point_on_two_calls():
    big = _case(1, B=8, H=32, C=4096, lens=[4096, 3000, 2049, 1025, 4000, 129, 1, 3333],
                K=3072, N=1024, n_add=70001)
    small = _case(2, B=2, H=8, C=1500, lens=[1500, 700], K=1024, N=3072, n_add=999)
    for name, (arrays, recs) in (("large", big), ("smaller", small)):
        descs_need = G.gpuos_eager_scratch_bytes(to_descs(recs, [1 << 40] * len(arrays)))
        say(f"{name} call: split partials need {descs_need} bytes of the static array")
        got = _run("static", arrays, recs)
        ref = _run("workspace", arrays, recs)
        for g, r, what in zip(got, ref, ("attention", "vector-matrix", "add")):
            assert np.array_equal(g, r), f"{name} call: {what} output differs"
