"""torch.library registration of libtq's entry points (no GPU needed): the ops
exist, their fake kernels give the right shapes and dtypes, seeds survive the
signed-int64 schema, and host tensors are refused (there is no CPU path)."""
import pytest
import torch

from kv_cache_vector_amd import torch_ops as T

OPS = torch.ops.kv_cache_vector


def test_ops_registered():
    for name in ("tq_encode", "tq_decode", "tq_encode_paged_", "tq_attn_decode"):
        assert hasattr(OPS, name), name


@pytest.mark.parametrize("bits,P", [(2, 32), (3, 48), (4, 64)])
def test_fake_shapes(bits, P):
    x = torch.empty(2, 7, 128, dtype=torch.float16, device="meta")
    packed, norms = OPS.tq_encode(x, bits, 0)
    assert packed.shape == (2, 7, P) and packed.dtype == torch.uint8
    assert norms.shape == (2, 7) and norms.dtype == torch.float32
    y = OPS.tq_decode(packed, norms, bits, 0)
    assert y.shape == (2, 7, 128) and y.dtype == torch.float16
    q = torch.empty(3, 8, 128, dtype=torch.float16, device="meta")
    kp = torch.empty(10, 16, 2, P, dtype=torch.uint8, device="meta")
    kn = torch.empty(10, 16, 2, dtype=torch.float32, device="meta")
    bt = torch.empty(3, 4, dtype=torch.int32, device="meta")
    cl = torch.empty(3, dtype=torch.int32, device="meta")
    o = OPS.tq_attn_decode(q, kp, kn, kp, kn, bt, cl, bits, 0, 0.088)
    assert o.shape == q.shape and o.dtype == torch.float16


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_fake_shapes_other_head_dims(d, bits):
    x = torch.empty(5, d, dtype=torch.float16, device="meta")
    packed, norms = OPS.tq_encode(x, bits, 0)
    assert packed.shape == (5, d * bits // 8) and norms.shape == (5,)
    y = OPS.tq_decode(packed, norms, bits, 0)
    assert y.shape == (5, d) and y.dtype == torch.float16


def test_fake_rejects_unsupported_head_dims():
    for d in (32, 96, 512):
        x = torch.empty(4, d, dtype=torch.float16, device="meta")
        with pytest.raises(ValueError):
            OPS.tq_encode(x, 4, 0)
    with pytest.raises(ValueError):                     # 20 bytes of 4-bit codes: d = 40
        OPS.tq_decode(torch.empty(4, 20, dtype=torch.uint8, device="meta"),
                      torch.empty(4, dtype=torch.float32, device="meta"), 4, 0)


def test_fake_rejects_unsupported_bits():
    x = torch.empty(4, 128, dtype=torch.float16, device="meta")
    with pytest.raises(ValueError):
        OPS.tq_encode(x, 5, 0)


def test_seed_round_trip():
    for s in (0, 42, 2 ** 63 - 1, 2 ** 63, 2 ** 64 - 1):
        v = T.seed_to_i64(s)
        assert -(2 ** 63) <= v < 2 ** 63
        assert v % (2 ** 64) == s


def test_host_tensors_refused():
    x = torch.zeros(4, 128, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        OPS.tq_encode(x, 4, 0)


def _attn_args(device="meta", P=64, **over):
    a = dict(query=torch.empty(3, 8, 128, dtype=torch.float16, device=device),
             k_packed=torch.empty(10, 16, 2, P, dtype=torch.uint8, device=device),
             k_norms=torch.empty(10, 16, 2, dtype=torch.float32, device=device),
             v_packed=torch.empty(10, 16, 2, P, dtype=torch.uint8, device=device),
             v_norms=torch.empty(10, 16, 2, dtype=torch.float32, device=device),
             block_tables=torch.empty(3, 4, dtype=torch.int32, device=device),
             context_lens=torch.empty(3, dtype=torch.int32, device=device))
    a.update(over)
    return a


def _paged_attention():
    from kv_cache_vector_amd.turboquant import TQPagedAttention, TurboQuant
    return TQPagedAttention(TurboQuant(128, 4, 0, "cuda"), 8)


def test_paged_attention_valid_arguments_reach_the_launch():
    """Valid (meta) arguments pass every check and stop only at the GPU
    requirement, i.e. at the launch itself."""
    attn = _paged_attention()
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.forward(**_attn_args())
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.forward(**_attn_args(), out=torch.empty(3, 8, 128, dtype=torch.float16,
                                                     device="meta"))


@pytest.mark.parametrize("bad", [
    dict(out=torch.empty(3, 8, 64, dtype=torch.float16, device="meta")),        # short
    dict(out=torch.empty(3, 8, 128, dtype=torch.float32, device="meta")),       # dtype
    dict(out=torch.empty(3, 128, 8, dtype=torch.float16, device="meta").transpose(1, 2)),
    dict(out=torch.empty(3, 8, 128, dtype=torch.float16, device="cpu")),        # device
    dict(k_norms=torch.empty(10, 16, 2, dtype=torch.float16, device="meta")),
    dict(v_norms=torch.empty(10, 16, 2, dtype=torch.float16, device="meta")),
    dict(k_packed=torch.empty(10, 16, 2, 64, dtype=torch.int8, device="meta")),
    dict(v_packed=torch.empty(10, 16, 2, 32, dtype=torch.uint8, device="meta")),
    dict(block_tables=torch.empty(3, 4, dtype=torch.int64, device="meta")),
    dict(context_lens=torch.empty(4, dtype=torch.int32, device="meta")),
    dict(block_tables=torch.empty(3, 4, dtype=torch.int32, device="cpu")),      # device
    dict(query=torch.empty(3, 8, 128, dtype=torch.float32, device="meta")),
    dict(query=torch.empty(3, 4, 128, dtype=torch.float16, device="meta")),     # heads
])
def test_paged_attention_rejects_bad_arguments_before_launch(bad):
    """Each bad argument raises a ValueError naming it, never the GPU
    requirement (the check runs before anything reaches libtq)."""
    attn = _paged_attention()
    args = _attn_args()
    out = bad.pop("out", None)
    args.update(bad)
    with pytest.raises(ValueError) as e:
        attn.forward(**args, out=out)
    assert "GPU tensor" not in str(e.value)


def test_attention_op_fake_checks_arguments():
    a = _attn_args()
    a["k_norms"] = torch.empty(10, 16, 2, dtype=torch.float16, device="meta")
    with pytest.raises(ValueError, match="float32"):
        OPS.tq_attn_decode(*a.values(), 4, 0, 0.088)


def test_hybrid_ops_fake_shapes_and_checks():
    from kv_cache_vector_amd.turboquant import HybridTurboQuant
    x = torch.empty(3, 5, 128, dtype=torch.float16, device="meta")
    perm = torch.arange(128, dtype=torch.int32)
    for mode, row in ((35, 68), (25, 52)):
        p = OPS.tq_hybrid_encode(x, mode, 0, perm)
        assert p.shape == (3, 5, row) and p.dtype == torch.uint8
        y = OPS.tq_hybrid_decode(p, mode, 0, perm)
        assert y.shape == (3, 5, 128) and y.dtype == torch.float16
    with pytest.raises(ValueError):
        OPS.tq_hybrid_encode(x, 40, 0, perm)
    with pytest.raises(ValueError):
        OPS.tq_hybrid_decode(torch.empty(4, 60, dtype=torch.uint8, device="meta"), 35, 0, perm)
    with pytest.raises(ValueError, match="GPU"):
        OPS.tq_hybrid_encode(torch.zeros(2, 128, dtype=torch.float16), 35, 0, perm)
    assert HybridTurboQuant.packed_dim_for_mode(128, "tq35") == 68
    assert HybridTurboQuant.packed_dim_for_mode(128, "tq25") == 52
    assert HybridTurboQuant.packed_dim_for_mode(64, "tq35") == 0
    h = HybridTurboQuant(128, "tq25", 1, "cuda")
    assert abs(h.compression_ratio() - 256 / 52) < 1e-12
    # calibration (host statistics): the 64 channels of largest mean square form group A
    scale = torch.ones(128)
    scale[[3, 70, 127]] = 20.0
    h.calibrate(torch.randn(2000, 128) * scale)
    assert {3, 70, 127} <= set(h.perm[:64].tolist())
    assert sorted(h.perm.tolist()) == list(range(128))
    h.calibrate_uniform(8)
    assert h.perm.tolist() == list(range(128)) and h.num_kv_heads == 8


def test_verify_slots_rejects_what_the_paged_write_assumes_away():
    """The paged write's slot contract: non-negative slots distinct and in
    range, negative ones skipped (checked on the host, opt-in)."""
    import torch
    from kv_cache_vector_amd.turboquant import verify_slots
    verify_slots(torch.tensor([3, 0, 7, -1, -1], dtype=torch.int64), 8)
    verify_slots(torch.tensor([-1, -5], dtype=torch.int64), 8)
    verify_slots(torch.tensor([], dtype=torch.int64), 8)
    with pytest.raises(ValueError, match="past the cache"):
        verify_slots(torch.tensor([1, 8], dtype=torch.int64), 8)
    with pytest.raises(ValueError, match="distinct"):
        verify_slots(torch.tensor([2, 5, 2], dtype=torch.int64), 8)
