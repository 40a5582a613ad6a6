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
