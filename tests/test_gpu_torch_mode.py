"""GPU parity of the PyTorch routing layer (torch_mode.GpuosMode): eager
aten calls inside the mode run on the persistent executor through the C
ABI, with normal launches mixed in, and agree with the oracle."""
import numpy as np
import pytest

import workloads as W
import oracle
from gpu_harness import check_outputs, run_record_oracle, say
from oracle_util import rec

pytestmark = pytest.mark.gpu


def test_routed_sequence_matches_the_oracle():
    import torch
    import torch.nn.functional as F
    from persistent_micro_dispatch_amd import gpuos as G
    from persistent_micro_dispatch_amd.torch_mode import GpuosMode, RoutingFilter

    gen = torch.Generator(device="cpu").manual_seed(7)
    xh = torch.randn(4, 1024, generator=gen)
    wh = torch.randn(4, 1024, generator=gen)
    x, w = xh.cuda(), wh.cuda()
    torch.cuda.current_stream().synchronize()
    with GpuosMode(filter=RoutingFilter(hot_after=1), ring_entries=64) as m:
        y0 = x * w
        y1 = y0 + x
        z = torch.relu(y1)
        g = F.gelu(z, approximate="tanh")
        s = torch.softmax(g, -1)
        t = s.sum(-1)
        mx = g.amax(-1)
        x.add_(z)
        cache = torch.zeros(8, 1024, device="cuda")   # a normal launch
        cache[2].copy_(g[1])                            # cache update, routed after the zeros
        st = G.gpuos_stats_get(m.ctx)
    say(f"routed {dict(m.stats.routed)}, normal {dict(m.stats.fallback)}, submitted {st['submitted']}")
    assert st["submitted"] == 9 and sum(m.stats.routed.values()) == 9
    # the same sequence as oracle records
    f4 = lambda n: np.zeros(n, np.float32)  # noqa: E731
    arrays = [xh.numpy().reshape(-1).copy(), wh.numpy().reshape(-1).copy(), f4(4096), f4(4096), f4(4096),
              f4(4096), f4(4096), f4(4), f4(4), f4(8 * 1024)]
    X, Wb, Y0, Y1, Z, Gb, S, T, MX, CA = range(10)
    n = 4096
    recs = np.concatenate([
        rec(W.OP_MUL, size=n, a=X, b=Wb, out=Y0), rec(W.OP_ADD, size=n, a=Y0, b=X, out=Y1),
        rec(W.OP_RELU, size=n, a=Y1, out=Z), rec(W.OP_GELU, size=n, a=Z, out=Gb),
        rec(W.OP_SOFTMAX, size=4, dim=(1024,), a=Gb, out=S), rec(W.OP_SUM, size=4, dim=(1024,), a=S, out=T),
        rec(W.OP_MAX, size=4, dim=(1024,), a=Gb, out=MX), rec(W.OP_ADD, size=n, a=X, b=Z, out=X),
        rec(W.OP_COPY, size=4096, a=(Gb, 4096), out=(CA, 2 * 4096)),
    ])
    # teacher-forced replay: each record runs on the oracle from the GPU's
    # values of its inputs (the pool adopts every GPU output after its
    # record), so exact ops compare bit for bit from identical inputs; no
    # later record overwrites an earlier one's output here, so the final GPU
    # tensors hold every record's output
    gpu = [t_.detach().cpu().numpy().reshape(-1).view(np.uint8) for t_ in (x, w, y0, y1, z, g, s, t, mx, cache)]
    pool = oracle.Pool([a.copy() for a in arrays])
    for k, r in enumerate(recs):
        hp = run_record_oracle(pool, r, False)
        pairs = [(gpu[b][o: o + nb], pool.arrays[b][o: o + nb]) for (b, o, nb) in W.output_ranges(r)]
        res = check_outputs(r, pool.arrays, pairs, hp)
        assert res["ok"], (k, res)
        say(f"  {res['op']}: worst error ratio {res['worst']:.3g}")
        for (b, o, nb) in W.output_ranges(r):
            pool.arrays[b][o: o + nb] = gpu[b][o: o + nb]


def test_hybrid_loop_matches_plain_pytorch():
    """A loop of small blocks in the mode with the default filter: each key is
    routed from its second sighting on, a matmul always takes the normal path,
    and the results equal plain PyTorch (exact ops bit for bit, GELU and
    softmax within their tolerances)."""
    import torch
    import torch.nn.functional as F
    from persistent_micro_dispatch_amd.torch_mode import GpuosMode

    gen = torch.Generator(device="cpu").manual_seed(3)
    a0 = torch.randn(16, 512, generator=gen).cuda()
    b0 = torch.randn(16, 512, generator=gen).cuda()
    wm = (torch.randn(512, 512, generator=gen) * 0.05).cuda()

    def block(a, b):
        h = torch.relu(a * b)
        h = h + a
        p = torch.softmax(F.gelu(h, approximate="tanh"), -1)
        q = (p @ wm)                      # a matmul: never routed
        return h, p, q, p.amax(-1)

    def run():
        out = []
        a, b = a0.clone(), b0.clone()
        for _ in range(20):
            h, p, q, mx = block(a, b)
            out.append((h.cpu(), p.cpu(), q.cpu(), mx.cpu()))
            a, b = p * 512.0, torch.relu(q) + b0   # bounded from one iteration to the next
        return out

    ref = run()
    torch.cuda.current_stream().synchronize()
    with GpuosMode(ring_entries=128) as m:
        got = run()
    say(f"routed {dict(m.stats.routed)}, normal {dict(m.stats.fallback)}")
    assert sum(m.stats.routed.values()) >= 100 and m.stats.fallback["op type"] >= 20
    for it, ((h, p, q, mx), (h2, p2, q2, mx2)) in enumerate(zip(ref, got)):
        # each iteration's inputs come from the previous one, computed on two
        # paths: the tolerance covers GELU/softmax rounding carried along
        assert torch.allclose(h2, h, rtol=1e-4, atol=1e-5), it
        assert torch.allclose(p2, p, rtol=1e-4, atol=1e-8), it
        assert torch.allclose(q2, q, rtol=1e-4, atol=1e-6), it
        assert torch.allclose(mx2, mx, rtol=1e-4, atol=1e-8), it


def test_linear_layers_route_to_the_matrix_cores():
    """F.linear without bias on bf16 activations of up to 64 rows runs as the
    executor's small matmul; results agree with torch's own bf16 matmul."""
    import torch
    import torch.nn.functional as F
    from persistent_micro_dispatch_amd.torch_mode import GpuosMode, RoutingFilter

    gen = torch.Generator(device="cpu").manual_seed(11)
    xs = [torch.randn(m, 1024, generator=gen).to(torch.bfloat16).cuda() for m in (1, 16, 64)]
    w = (torch.randn(3072, 1024, generator=gen) * 0.02).to(torch.bfloat16).cuda()
    ref = [F.linear(x, w).float().cpu() for x in xs]
    torch.cuda.current_stream().synchronize()
    with GpuosMode(filter=RoutingFilter(hot_after=1)) as m:
        got = [F.linear(x, w) for x in xs]
        got = [g.float().cpu() for g in got]
    say(f"routed {dict(m.stats.routed)}, normal {dict(m.stats.fallback)}")
    assert m.stats.routed["small matmul"] == 3
    for g, r in zip(got, ref):
        # two bf16 roundings of the same fp32-accumulated sums
        assert torch.allclose(g, r, rtol=2 ** -7, atol=2e-3)
