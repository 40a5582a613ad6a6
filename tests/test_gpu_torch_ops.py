"""The torch custom operators on the GPU: same bytes as the class API, the
paged write mutates the cache in place, and torch.compile traces a decode
step (paged write + attention) with fullgraph=True, i.e. without a graph
break."""
import math

import numpy as np
import pytest
import torch

from kv_cache_vector_amd import _lib
from kv_cache_vector_amd import torch_ops as T
from kv_cache_vector_amd import workloads as W
from kv_cache_vector_amd.turboquant import TQPagedAttention, TurboQuant

pytestmark = pytest.mark.gpu
OPS = torch.ops.kv_cache_vector


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an AMD Instinct GPU"
    _lib.load()
    return torch.device("cuda:0")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_ops_match_direct_calls(dev, d):
    print("[ops] encode/decode vs direct, d=%d" % d, flush=True)
    x = torch.from_numpy(W.gaussian(4096, seed=3, head_dim=d)).to(dev)
    seed = 2 ** 64 - 5                                   # needs the int64 conversion
    for bits in (2, 3, 4):
        p1, n1 = OPS.tq_encode(x, bits, T.seed_to_i64(seed))
        P = d * bits // 8
        assert p1.shape == (4096, P)
        p2 = torch.empty(4096, P, dtype=torch.uint8, device=dev)
        n2 = torch.empty(4096, dtype=torch.float32, device=dev)
        s = torch.cuda.current_stream().cuda_stream
        _lib.check(_lib.tq_encode(x.data_ptr(), 4096, d, bits, seed, p2.data_ptr(),
                                  n2.data_ptr(), s), "tq_encode")
        y1 = OPS.tq_decode(p1, n1, bits, T.seed_to_i64(seed))
        y2 = torch.empty_like(x)
        _lib.check(_lib.tq_decode(p2.data_ptr(), n2.data_ptr(), 4096, d, bits, seed,
                                  y2.data_ptr(), s), "tq_decode")
        torch.cuda.synchronize()
        assert torch.equal(p1, p2) and torch.equal(n1, n2) and torch.equal(y1, y2)


def _decode_step_inputs(dev):
    """A small paged cache, a query and one new token's K/V per sequence,
    with the slots of that token."""
    B, Hq, Hkv, T_ctx, bits, seed = 2, 8, 2, 40, 4, 7
    wl = W.attn_workload(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, context=T_ctx, seed=11,
                         perm_seed=12, ragged=False)
    tq = TurboQuant(128, bits, seed, dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    kp, kn = tq.encode(t(wl["k"]).reshape(-1, 128))
    vp, vn = tq.encode(t(wl["v"]).reshape(-1, 128))
    nblk = wl["k"].shape[0]
    kp, kn = kp.view(nblk, 16, Hkv, 64), kn.view(nblk, 16, Hkv)
    vp, vn = vp.view(nblk, 16, Hkv, 64), vn.view(nblk, 16, Hkv)
    bt, cl = t(wl["block_tables"]), t(wl["context_lens"])
    q = t(wl["q"])
    newk = torch.randn(B * Hkv, 128, device=dev).half()
    newv = torch.randn(B * Hkv, 128, device=dev).half()
    # the new token sits at position T_ctx - 1 of each sequence
    pos = T_ctx - 1
    blk = bt[:, pos // 16].long()
    slots = ((blk * 16 + pos % 16)[:, None] * Hkv + torch.arange(Hkv, device=dev)).reshape(-1)
    scale = 1 / math.sqrt(128)

    def step(q, newk, newv, kp, kn, vp, vn):
        OPS.tq_encode_paged_(newk, slots, kp, kn, bits, seed)
        OPS.tq_encode_paged_(newv, slots, vp, vn, bits, seed)
        return OPS.tq_attn_decode(q, kp, kn, vp, vn, bt, cl, bits, seed, scale)

    return dict(tq=tq, q=q, newk=newk, newv=newv, caches=(kp, kn, vp, vn), bt=bt, cl=cl,
                slots=slots, scale=scale, Hq=Hq, bits=bits, seed=seed, step=step)


def test_compiled_decode_step(dev):
    """Encode the new token's K/V into its cache slots, then attend; the
    compiled function must equal the eager one."""
    print("[ops] torch.compile fullgraph decode step", flush=True)
    inp = _decode_step_inputs(dev)
    tq, q, newk, newv, step = inp["tq"], inp["q"], inp["newk"], inp["newv"], inp["step"]
    kp, kn, vp, vn = inp["caches"]
    bt, cl, slots, scale, Hq = inp["bt"], inp["cl"], inp["slots"], inp["scale"], inp["Hq"]
    caches = [c.clone() for c in (kp, kn, vp, vn)]
    eager = step(q, newk, newv, *caches)
    compiled = torch.compile(step, backend="aot_eager", fullgraph=True)
    caches2 = [c.clone() for c in (kp, kn, vp, vn)]
    got = compiled(q, newk, newv, *caches2)
    torch.cuda.synchronize()
    assert torch.equal(got, eager)
    for a, b in zip(caches, caches2):
        assert torch.equal(a, b)
    # the written rows decode to the new vectors' codec round trip
    rows = tq.decode(caches2[0].view(-1, 64)[slots], caches2[1].view(-1)[slots])
    ref = tq.decode(*tq.encode(newk))
    assert torch.equal(rows, ref)
    # the class API gives the same attention
    attn = TQPagedAttention(tq, Hq, scale=scale)
    assert torch.equal(attn.forward(q, *caches2[:2], *caches2[2:], bt, cl), got)


def test_graph_captured_decode_step(dev):
    """The decode step (paged write of K and V, then attention) captured in a
    HIP graph: libtq allocates nothing and issues no memset, and the operators
    take their outputs and workspace from torch's allocator, so the captured
    step replays.  Every replay, with eager work and synchronisations between
    replays, must equal the eager step bit for bit."""
    print("[ops] graph-captured decode step", flush=True)
    inp = _decode_step_inputs(dev)
    q, newk, newv, step = inp["q"], inp["newk"], inp["newv"], inp["step"]
    init = [c.clone() for c in inp["caches"]]
    eager_caches = [c.clone() for c in init]
    eager = step(q, newk, newv, *eager_caches)
    torch.cuda.synchronize()

    caches = [c.clone() for c in init]          # the graph's static cache tensors
    side = torch.cuda.Stream()                  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):                      # warm-up outside the capture
            step(q, newk, newv, *caches)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step(q, newk, newv, *caches)
    torch.cuda.synchronize()

    other_q = torch.randn_like(q)
    for rep in range(4):
        for c, c0 in zip(caches, init):         # eager work: reset the cache
            c.copy_(c0)
        # unrelated eager work on the same stream between replays
        OPS.tq_attn_decode(other_q, *init, inp["bt"], inp["cl"], inp["bits"], inp["seed"],
                           inp["scale"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d" % rep
        for a, b in zip(caches, eager_caches):
            assert torch.equal(a, b), "replay %d" % rep


def test_hybrid_ops_compile_without_graph_breaks(dev):
    """The hybrid modes' operators trace under torch.compile(fullgraph=True)
    and give the same bytes as eager calls (the pages: every mode registers
    custom ops for zero-graph-break decode)."""
    from kv_cache_vector_amd.turboquant import HybridTurboQuant
    x = torch.from_numpy(W.gaussian(1000, seed=12)).to(dev)
    for mode in ("tq35", "tq25"):
        h = HybridTurboQuant(128, mode, 4, dev)
        h.calibrate(x)
        perm = torch.from_numpy(h.perm)
        m = HybridTurboQuant.MODES[mode]

        def step(x, perm=perm, m=m):
            p = OPS.tq_hybrid_encode(x, m, 4, perm)
            return p, OPS.tq_hybrid_decode(p, m, 4, perm)

        p1, y1 = step(x)
        p2, y2 = torch.compile(step, fullgraph=True)(x)
        torch.cuda.synchronize()
        assert torch.equal(p1, p2) and torch.equal(y1, y2)
        assert torch.equal(p1, h.encode(x)) and torch.equal(y1, h.decode(p1))
