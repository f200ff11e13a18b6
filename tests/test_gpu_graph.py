"""HIP graph capture of the attention entry points (GPU).

The kernels allocate nothing, write no memory through memset nodes and never synchronise, so
a call can be captured into a HIP graph (torch.cuda.CUDAGraph on ROCm) and replayed. Each test
captures one call on static tensors; then, for several rounds, it writes new inputs eagerly,
synchronises, replays the graph, and checks every output against an eager call on the same
inputs. The same kernels run on the same data, so the two must agree bit for bit.
"""

import pytest
import torch

from exact_attention_06_amd import fa_bwd, fa_decode, fa_fwd, fa_fwd_ext, fa_fwd_fp8, fa_prep_fp8

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _randn(seed, *shape, dtype=torch.bfloat16):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype).cuda()


def _replay_check(name, make_inputs, call, rounds=3):
    say(f"graph {name}")
    static = make_inputs(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        call(*static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = call(*static)
    for r in range(1, rounds + 1):
        new = make_inputs(r)
        for t, n in zip(static, new):
            t.copy_(n)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = call(*new)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            if a is None:
                continue
            assert torch.equal(a, b), f"{name}: output {i} of replay {r} differs from the eager call"
        del new, ref


@pytest.mark.parametrize("d,causal,dtype", [(128, True, torch.bfloat16), (64, False, torch.bfloat16),
                                            (256, True, torch.bfloat16), (64, True, torch.float32)])
def test_graph_fwd(d, causal, dtype):
    n = 700 if dtype == torch.bfloat16 else 200
    _replay_check(f"fa_fwd d={d} causal={causal} {dtype}",
                  lambda r: [_randn(100 * r + i, 2, 3, n, d, dtype=dtype) for i in range(3)],
                  lambda q, k, v: fa_fwd(q, k, v, causal=causal))


def test_graph_fwd_ext_packed():
    cu = torch.tensor([0, 300, 300, 1300, 2048], dtype=torch.int32).cuda()
    _replay_check("fa_fwd_ext packed, grouped heads, window",
                  lambda r: [_randn(10 * r, 1, 8, 2048, 128), _randn(10 * r + 1, 1, 2, 2048, 128),
                             _randn(10 * r + 2, 1, 2, 2048, 128)],
                  lambda q, k, v: fa_fwd_ext(q, k, v, causal=True, window=(255, 0), cu_seqlens=cu, max_seqlen=1000))


def test_graph_decode():
    _replay_check("fa_decode",
                  lambda r: [_randn(20 * r, 2, 8, 3, 128), _randn(20 * r + 1, 2, 2, 5000, 128),
                             _randn(20 * r + 2, 2, 2, 5000, 128)],
                  lambda q, k, v: fa_decode(q, k, v, causal=True))


def test_graph_bwd():
    def inputs(r):
        q, k, v, do = (_randn(30 * r + i, 1, 2, 600, 128) for i in range(4))
        o, lse = fa_fwd(q, k, v, causal=True)
        return [q, k, v, o, do, lse]

    _replay_check("fa_bwd", inputs, lambda q, k, v, o, do, lse: fa_bwd(q, k, v, o, do, lse, causal=True))


def test_graph_fp8_path():
    signs = (torch.randint(0, 2, (128,), generator=torch.Generator("cpu").manual_seed(3)) * 2 - 1).float().cuda()

    def path(q, k, v):
        q8, sq = fa_prep_fp8(q, signs)
        k8, sk = fa_prep_fp8(k, signs)
        v8, sv = fa_prep_fp8(v)
        o, lse = fa_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=False)
        return [q8, sq, k8, sk, v8, sv, o, lse]

    _replay_check("fa_prep_fp8 + fa_fwd_fp8",
                  lambda r: [_randn(40 * r + i, 1, 2, 1024, 128, dtype=torch.float32) for i in range(3)], path)
