"""The Python binding checks every tensor it hands to the C ABI (dtype, shape,
layout, device) and raises before any library call: the ABI receives bare
pointers and sizes, so a mismatch there would read or write out of bounds.
Runs on the host: the library is replaced by a recorder, and every case
asserts that nothing reached it."""
import pytest
import torch

i8 = pytest.importorskip("int8_mixed_precision_rowwise_amd")


class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*args):
            self.calls.append(name)
            return 0
        return f


@pytest.fixture
def lib(monkeypatch):
    rec = _Recorder()
    monkeypatch.setattr(i8, "lib", rec)
    yield rec
    assert rec.calls == [] or all(c.endswith("_workspace_bytes") for c in rec.calls), rec.calls


bf, i8t, f32, u8 = torch.bfloat16, torch.int8, torch.float32, torch.uint8


def t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def test_quantize_rowwise_checks(lib):
    with pytest.raises(TypeError, match="bfloat16"):
        i8.quantize_rowwise(t(4, 8, dtype=f32))
    with pytest.raises(ValueError, match="2-D"):
        i8.quantize_rowwise(t(2, 4, 8))
    with pytest.raises(ValueError, match="shape"):
        i8.quantize_rowwise(t(4, 8), q=t(4, 9, dtype=i8t))
    with pytest.raises(TypeError, match="int8"):
        i8.quantize_rowwise(t(4, 8), q=t(4, 8, dtype=u8))
    with pytest.raises(ValueError, match="4 elements"):
        i8.quantize_rowwise(t(4, 8), scale=t(8, dtype=f32))
    with pytest.raises(ValueError, match="contiguous"):
        i8.quantize_rowwise(t(8, 4).t())  # columns strided
    with pytest.raises(ValueError, match="contiguous"):
        i8.quantize_rowwise(t(4, 8), scale=t(8, dtype=f32)[::2])
    with pytest.raises(ValueError, match="device tensors"):
        i8.quantize_rowwise(t(4, 8))  # right shapes, but host memory


def test_quantize_colwise_and_colmax_checks(lib):
    with pytest.raises(ValueError, match="8 elements"):
        i8.quantize_colwise(t(4, 8), scale=t(4, dtype=f32))
    with pytest.raises(TypeError, match="uint8"):
        i8.quantize_colwise(t(4, 8), workspace=t(64, dtype=f32))
    with pytest.raises(ValueError, match="8 elements"):
        i8.quantize_rowwise_colmax(t(4, 8), colmax=t(4, dtype=f32))
    with pytest.raises(ValueError, match="8 elements"):
        i8.quantize_colwise_given_colmax(t(4, 8), t(4, dtype=f32))
    with pytest.raises(TypeError, match="float32"):
        i8.quantize_colwise_given_colmax(t(4, 8), t(8, dtype=bf))
    with pytest.raises(ValueError, match="shape"):
        i8.quantize_colwise_given_colmax(t(4, 8), t(8, dtype=f32), q=t(8, 4, dtype=i8t))
    with pytest.raises(ValueError, match="one device"):
        i8.quantize_colwise_given_colmax(t(4, 8), torch.zeros(8, dtype=f32, device="meta"))


def test_gemm_checks(lib):
    A, B = t(4, 16, dtype=i8t), t(8, 16, dtype=i8t)
    sa, sb = t(4, dtype=f32), t(8, dtype=f32)
    with pytest.raises(ValueError, match="layout"):
        i8.int8_scaled_mm("TT", A, sa, B, sb)
    with pytest.raises(ValueError, match="do not match"):
        i8.int8_scaled_mm("NT", A, sa, t(8, 12, dtype=i8t), sb)
    with pytest.raises(ValueError, match="do not match"):
        i8.int8_scaled_mm("NN", A, sa, B, sb)  # B would need 16 rows
    with pytest.raises(ValueError, match="scale_a"):
        i8.int8_scaled_mm("NT", A, sb, B, sb)
    with pytest.raises(ValueError, match="scale_b"):
        i8.int8_scaled_mm("NT", A, sa, B, sa)
    with pytest.raises(TypeError, match="scale_a"):
        i8.int8_scaled_mm("NT", A, None, B, sb)
    with pytest.raises(TypeError, match="float32"):
        i8.int8_scaled_mm("NT", A, sa.double(), B, sb)
    with pytest.raises(ValueError, match="out"):
        i8.int8_scaled_mm("NT", A, sa, B, sb, out=t(8, 4))
    with pytest.raises(TypeError, match="out"):
        i8.int8_scaled_mm("NT", A, sa, B, sb, out=t(4, 8, dtype=f32))
    with pytest.raises(ValueError, match="out"):
        i8.int8_mm_i32("NT", A, B, out=t(4, 7, dtype=torch.int32))
    with pytest.raises(TypeError, match="int8"):
        i8.int8_mm_i32("NT", A.to(u8), B)
    with pytest.raises(TypeError, match="uint8"):
        i8.fp8_scaled_mm("NT", A, sa, B, sb)
    with pytest.raises(ValueError, match="device tensors"):
        i8.int8_scaled_mm("TN", t(16, 4, dtype=i8t), sa, t(16, 8, dtype=i8t), sb)


def test_linear_checks(lib):
    X, W, dY = t(6, 16), t(8, 16), t(6, 8)
    with pytest.raises(ValueError, match="16 columns"):
        i8.linear_fwd(X, t(8, 12))
    with pytest.raises(ValueError, match="contiguous"):
        i8.linear_fwd(t(6, 32)[:, :16], W)  # padded rows: the chains take ld = K
    with pytest.raises(ValueError, match="out"):
        i8.linear_fwd(X, W, out=t(8, 6))
    with pytest.raises(ValueError, match="contiguous"):
        i8.linear_fwd_colmax(X, W, out=t(6, 16)[:, :8])
    with pytest.raises(TypeError, match="uint8"):
        i8.linear_fwd(X, W, workspace=t(16, dtype=i8t))
    with pytest.raises(ValueError, match="8 rows"):
        i8.linear_bwd(dY, X, t(4, 16))
    with pytest.raises(ValueError, match="X"):
        i8.linear_bwd(dY, t(6, 12), W)
    with pytest.raises(ValueError, match="dX"):
        i8.linear_bwd(dY, X, W, dX=t(6, 8))
    with pytest.raises(ValueError, match="dW"):
        i8.linear_bwd(dY, X, W, dW=t(16, 8))
    with pytest.raises(ValueError, match="colmax_x"):
        i8.linear_bwd(dY, X, W, colmax_x=t(8, dtype=f32))
    with pytest.raises(ValueError, match="colmax_w"):
        i8.linear_bwd(dY, X, W, colmax_w=t(16, 1, dtype=f32))
    with pytest.raises(TypeError, match="bfloat16"):
        i8.linear_bwd_fp8(dY.float(), X, W)
    with pytest.raises(ValueError, match="device tensors"):
        i8.linear_bwd(dY, X, W)
    with pytest.raises(ValueError, match="n_blocks"):
        i8.philox4x32_10(0, 0, -1)
