"""The whole path (quantize Q and K, route, forward) captured in one HIP graph
and replayed: every replay must give exactly the eager results, with eager
work on the same device between replays, and new inputs copied into the
captured input tensors must give that input's eager results.  The path
allocates nothing and queues everything on the caller's stream, which is
what makes it capturable; its kernels are deterministic, so the comparison
is bit for bit."""
import pytest
import torch

import workloads as W
from tests.helpers import bf16_dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    import block_sparse_int8_amd as m
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    m.device_check(torch.cuda.current_device())
    return m


def _inputs(seed):
    wl = W.tiny_sol(seed=seed, H=2, L=1024, d=128, valid=1000)
    return bf16_dev(wl.q), bf16_dev(wl.k), bf16_dev(wl.v)


def _same(got, ref):
    return all(torch.equal(g, r) for g, r in zip(got, ref))


@pytest.mark.parametrize("rule", [0, 1])
def test_pipeline_graph_replay(sa, rule):
    say(f"case graph replay rule={rule}")
    kw = dict(lq_valid=1000, lkv_valid=1000, threshold=1.0, centroids_per_block=1, rule=rule, sparsity=0.6,
              out_dtype=torch.bfloat16, return_lse=True)
    q, k, v = _inputs(71)
    q2, k2, v2 = _inputs(72)

    def run(a, b, c):
        (out, lse), bmap = sa.sparse_attention(a, b, c, **kw)
        return out, lse, bmap

    ref1 = [t.clone() for t in run(q, k, v)]
    ref2 = [t.clone() for t in run(q2, k2, v2)]
    torch.cuda.synchronize()
    assert not _same(ref1, ref2)

    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(q, k, v)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = run(q, k, v)

    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert _same(captured, ref1), f"replay {rep} differs from the eager run"
        eager = run(q2, k2, v2)          # other work between replays
        torch.cuda.synchronize()
        assert _same(eager, ref2)

    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    g.replay()
    torch.cuda.synchronize()
    assert _same(captured, ref2), "replay on new inputs differs from their eager run"


@pytest.mark.parametrize("rule", [0, 1])
def test_pipeline_on_a_side_stream(sa, rule):
    """The whole path queued on a stream other than torch's current one: the
    binding records that stream on every tensor it allocates, so memory the
    caching allocator hands out on the current stream right after the call
    returns (before the side stream has run) is not memory the kernels still
    use.  The result must equal the current-stream run bit for bit."""
    say(f"case side stream rule={rule}")
    kw = dict(lq_valid=1000, lkv_valid=1000, threshold=1.0, centroids_per_block=1, rule=rule, sparsity=0.6,
              out_dtype=torch.float32, return_lse=True)
    q, k, v = _inputs(73)
    (ref_out, ref_lse), ref_map = sa.sparse_attention(q, k, v, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    hold = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    torch.cuda._sleep(50_000_000)                 # keep the side stream's work queued behind the sleep
    side.wait_stream(torch.cuda.current_stream())
    (out, lse), bmap = sa.sparse_attention(q, k, v, stream=side, **kw)
    # while the side stream waits: allocate and fill on the current stream
    junk = [torch.full((1 << 20,), float(i), device="cuda") for i in range(16)]
    del junk, hold
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse) and torch.equal(bmap, ref_map)
