"""The Python layer above the C ABI refuses malformed arguments loudly, before any kernel runs: the dtype, shape,
layout and device of the inputs, of the optional key-padding lengths and output buffers, and of the fp8 and
packed entry points' inputs. A size the C ABI itself refuses (head dim 96) comes back as RuntimeError."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_13_amd as fa_mod
    return fa_mod


def _t(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_forward_rejects_malformed_arguments(fa):
    q = _t((1, 2, 64, 64))
    print("[case] forward argument checks", flush=True)
    with pytest.raises(TypeError):
        fa.forward(q.float(), q, q)  # mixed dtypes
    with pytest.raises(TypeError):
        fa.forward(q.half(), q.half(), q.half())  # fp16 is not an input type
    with pytest.raises(ValueError):
        fa.forward(q.transpose(2, 3), q, q)  # not row-major
    with pytest.raises(ValueError):
        fa.forward(q[0], q[0], q[0])  # not [B, H, N, d]
    with pytest.raises(ValueError):
        fa.forward(q, _t((1, 3, 64, 64)), _t((1, 3, 64, 64)))  # H_kv does not divide H
    with pytest.raises(ValueError):
        fa.forward(q, q, _t((1, 2, 32, 64)))  # v of another length
    q32 = q.float()
    with pytest.raises(TypeError):
        fa.forward(q32, _t((1, 1, 64, 64), torch.float32), _t((1, 1, 64, 64), torch.float32))  # grouped heads in fp32
    with pytest.raises(ValueError):
        fa.forward(q, q, q, kv_len=torch.tensor([64], dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError):
        fa.forward(q, q, q, kv_len=torch.tensor([64, 64], dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        fa.forward(q, q, q, out=_t((1, 2, 64, 64), torch.float32))
    with pytest.raises(ValueError):
        fa.forward(q, q, q, lse=_t((1, 2, 64), torch.bfloat16))
    d96 = _t((1, 1, 64, 96))
    with pytest.raises(RuntimeError):
        fa.forward(d96, d96, d96)


def test_backward_rejects_malformed_arguments(fa):
    q = _t((1, 2, 64, 64))
    lse = _t((1, 2, 64), torch.float32)
    print("[case] backward argument checks", flush=True)
    with pytest.raises(TypeError):
        fa.backward(q.float(), q.float(), q.float(), q.float(), lse, q.float())  # fp32 has no gradient kernel
    with pytest.raises(ValueError):
        fa.backward(q, q, q, _t((1, 2, 32, 64)), lse, q)  # o of another shape
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse, q.transpose(2, 3))  # dout not row-major
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, _t((1, 2, 64)), q)  # lse not fp32
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse, q, kv_len=torch.tensor([1.0], device="cuda"))


def test_fp8_and_packed_entry_points_reject_malformed_arguments(fa):
    print("[case] fp8 and packed argument checks", flush=True)
    q8 = _t((1, 2, 64, 64), torch.float8_e4m3fn)
    vt8 = _t((1, 2, 64, 64), torch.float8_e4m3fn)
    with pytest.raises(TypeError):
        fa.forward_fp8(q8.to(torch.bfloat16), q8, vt8, 1.0, 1.0, 1.0)  # q not fp8
    with pytest.raises(ValueError):
        fa.forward_fp8(q8, q8, _t((1, 2, 64, 32), torch.float8_e4m3fn), 1.0, 1.0, 1.0)  # vt not [B, H, d, N]
    qp = _t((100, 2, 64))
    cu = torch.tensor([0, 60, 100], dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):
        fa.forward_varlen(qp.float(), qp.float(), qp.float(), cu, 60)  # packed inputs are bf16
    with pytest.raises(ValueError):
        fa.forward_varlen(qp, qp, qp, cu.long(), 60)  # offsets not int32
    with pytest.raises(ValueError):
        fa.forward_varlen(qp, _t((100, 3, 64)), _t((100, 3, 64)), cu, 60)  # H_kv does not divide H
    lse = _t((2, 100), torch.float32)
    with pytest.raises(ValueError):
        fa.backward_varlen(qp, qp, qp, qp, _t((100, 2), torch.float32), qp, cu, 60)  # lse not [H, total]
    with pytest.raises(ValueError):
        fa.backward_varlen(qp, qp, qp, _t((99, 2, 64)), lse, qp, cu, 60)  # o of another length
