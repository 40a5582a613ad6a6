"""tq_attn_decode_kv_noalloc: the attention entry point that allocates
nothing (its workspace is the library's fixed per-GPU array) gives the same
bytes as tq_attn_decode_kv with a caller's workspace, on two calls in a row,
the second smaller than the first."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import parity as P
from kv_cache_vector_amd import _lib
from kv_cache_vector_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an AMD Instinct GPU"
    _lib.load()
    return torch.device("cuda:0")


def _case(dev, B, Hq, Hkv, T, kb, vb, d, seed):
    wl = W.attn_workload(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, context=T, seed=seed,
                         perm_seed=seed + 1, ragged=True, head_dim=d)
    kp, kn = oracle.encode(wl["k"], kb, 0)
    vp, vn = oracle.encode(wl["v"], vb, 0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return dict(wl=wl, host=(kp, kn, vp, vn),
                dev=[t(a) for a in (wl["q"], kp, kn, vp, vn, wl["block_tables"],
                                    wl["context_lens"])])


def _args(c, B, Hq, Hkv, d, kb, vb):
    q, kp, kn, vp, vn, bt, cl = c["dev"]
    maxb = bt.shape[1]
    return (q.data_ptr(), kp.data_ptr(), kn.data_ptr(), vp.data_ptr(), vn.data_ptr(),
            bt.data_ptr(), cl.data_ptr(), B, Hq, Hkv, d, kb, vb, 0, 16, maxb, kp.shape[0],
            1 / math.sqrt(d))


def test_no_alloc_matches_workspace_entry_point(dev):
    s = torch.cuda.current_stream().cuda_stream
    # first a larger call, then a smaller one: the shared array keeps the
    # first call's contents, which the second must not depend on
    shapes = [(8, 32, 8, 3000, 4, 4, 128, 41), (3, 8, 2, 300, 4, 2, 128, 43)]
    for (B, Hq, Hkv, T, kb, vb, d, seed) in shapes:
        P.log("[no-alloc] B=%d Hq=%d Hkv=%d T=%d bits %d/%d d=%d" % (B, Hq, Hkv, T, kb, vb, d))
        c = _case(dev, B, Hq, Hkv, T, kb, vb, d, seed)
        a = _args(c, B, Hq, Hkv, d, kb, vb)
        need = _lib.tq_attn_workspace_bytes(B, Hq, Hkv, d, 16, c["dev"][5].shape[1])
        assert 0 < need <= _lib.TQ_ATTN_NOALLOC_WORKSPACE_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        ref = torch.empty(B, Hq, d, dtype=torch.float16, device=dev)
        out = torch.full((B, Hq, d), 7.0, dtype=torch.float16, device=dev)
        _lib.check(_lib.tq_attn_decode_kv(*a, ref.data_ptr(), ws.data_ptr(), need, s),
                   "tq_attn_decode_kv")
        _lib.check(_lib.tq_attn_decode_kv_noalloc(*a, out.data_ptr(), s),
                   "tq_attn_decode_kv_noalloc")
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        # and both against the oracle
        wl = c["wl"]
        kp, kn, vp, vn = c["host"]
        _, exact = oracle.attn_decode(wl["q"], kp, kn, vp, vn, wl["block_tables"],
                                      wl["context_lens"], Hkv, kb, 0, 1 / math.sqrt(d),
                                      want_f64=True, v_bits=vb)
        P.compare_attn(out.cpu().numpy(), exact, "no-alloc")


def test_no_alloc_rejects_shapes_beyond_its_array(dev):
    """A shape whose workspace exceeds the fixed array returns
    TQ_ERR_WORKSPACE before anything is launched."""
    s = torch.cuda.current_stream().cuda_stream
    B, Hq, Hkv, d = 512, 64, 8, 128
    maxb = 1024                                   # 16K tokens per sequence
    need = _lib.tq_attn_workspace_bytes(B, Hq, Hkv, d, 16, maxb)
    assert need > _lib.TQ_ATTN_NOALLOC_WORKSPACE_BYTES
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    p = buf.data_ptr()
    st = _lib.tq_attn_decode_kv_noalloc(p, p + 4096, p + 8192, p + 12288, p + 16384,
                                        p + 20480, p + 24576, B, Hq, Hkv, d, 4, 4, 0, 16,
                                        maxb, 0, 0.088, p + 65536, s)
    assert st == 4                                # TQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(buf.sum()) == 0                    # nothing was written
