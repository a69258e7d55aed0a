"""GPU parity of the training integration.

* A 2-layer MLP (linear, ReLU, linear) swapped by ``swap_linear_modules``: its
  output and every gradient, bit for bit, against the oracle's linear chains
  (RNE and SR, each layer with its own Philox key).
* Each of the 8 INT8/BF16 choices of (forward, grad-input, grad-weight) on one
  layer: INT8 GEMMs against the oracle, BF16 ones against torch's bf16 matmul.
* Stochastic rounding advances its Philox offset by one step per forward call.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import tensor_bits
from workloads import gaussian_bf16

pytestmark = pytest.mark.gpu

i8 = pytest.importorskip("int8_mixed_precision_rowwise_amd")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
from int8_mixed_precision_rowwise_amd import training as T  # noqa: E402

RC = {"rne": oracle.RNE, "sr": oracle.SR}


def relu_bits(b: np.ndarray) -> np.ndarray:
    """bf16 ReLU on bit patterns: negative values and -0 become +0."""
    return np.where((b & 0x8000) != 0, 0, b).astype(np.uint16)


def positive_bits(b: np.ndarray) -> np.ndarray:
    return ((b & 0x8000) == 0) & (b != 0)


def same(t: torch.Tensor, bits: np.ndarray, what: str):
    got = tensor_bits(t).reshape(bits.shape)
    if not np.array_equal(got, bits):
        raise AssertionError(f"{what}: {int(np.count_nonzero(got != bits))} of {bits.size} differ")


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_mlp_output_and_gradients_match_oracle(rounding):
    B, S, K1, H, N = 2, 96, 512, 768, 320
    x = gaussian_bf16(B * S, K1, seed=1).view(B, S, K1).cuda().requires_grad_()
    W1 = gaussian_bf16(H, K1, seed=2, std=0.02)
    W2 = gaussian_bf16(N, H, seed=3, std=0.02)
    G = gaussian_bf16(B * S, N, seed=4, std=1e-3).view(B, S, N).cuda()
    model = torch.nn.Sequential(torch.nn.Linear(K1, H, bias=False), torch.nn.ReLU(),
                                torch.nn.Linear(H, N, bias=False)).to(torch.bfloat16).cuda()
    with torch.no_grad():
        model[0].weight.copy_(W1)
        model[2].weight.copy_(W2)
    T.swap_linear_modules(model, T.Int8MixedPrecisionConfig(stochastic_rounding=rounding == "sr", seed=77))
    y = model(x)
    y.backward(G)

    r, s1, s2 = RC[rounding], model[0].seed, model[2].seed
    Xb = tensor_bits(x.detach()).reshape(B * S, K1)
    W1b, W2b, Gb = tensor_bits(W1), tensor_bits(W2), tensor_bits(G).reshape(B * S, N)
    Y1 = oracle.linear_fwd(Xb, W1b, r, s1, 0)
    Hb = relu_bits(Y1)
    Y2 = oracle.linear_fwd(Hb, W2b, r, s2, 0)
    dH, dW2 = oracle.linear_bwd(Gb, Hb, W2b, r, s2, 0)
    dY1 = np.where(positive_bits(Y1), dH, 0).astype(np.uint16)
    dX, dW1 = oracle.linear_bwd(dY1, Xb, W1b, r, s1, 0)
    same(y, Y2, "y")
    same(x.grad, dX, "dX")
    same(model[0].weight.grad, dW1, "dW1")
    same(model[2].weight.grad, dW2, "dW2")


def test_per_gemm_toggles():
    M, K, N = 256, 384, 192
    X = gaussian_bf16(M, K, seed=11).cuda()
    W = gaussian_bf16(N, K, seed=12, std=0.02).cuda()
    G = gaussian_bf16(M, N, seed=13, std=1e-3).cuda()
    Xb, Wb, Gb = tensor_bits(X), tensor_bits(W), tensor_bits(G)
    Yo = oracle.linear_fwd(Xb, Wb, oracle.RNE, 3, 0)
    dXo, dWo = oracle.linear_bwd(Gb, Xb, Wb, oracle.RNE, 3, 0)
    Yt, dXt, dWt = (tensor_bits(t) for t in (torch.mm(X, W.t()), torch.mm(G, W), torch.mm(G.t(), X)))
    assert not np.array_equal(Yo, Yt) and not np.array_equal(dXo, dXt) and not np.array_equal(dWo, dWt)
    for o, gi, gw in itertools.product([True, False], repeat=3):
        cfg = T.Int8MixedPrecisionConfig(output=o, grad_input=gi, grad_weight=gw)
        lin = T.Int8MixedPrecisionLinear(K, N, cfg, seed=3).cuda()
        with torch.no_grad():
            lin.weight.copy_(W)
        x = X.clone().requires_grad_()
        y = lin(x)
        y.backward(G)
        tag = f"output={o} grad_input={gi} grad_weight={gw}"
        same(y, Yo if o else Yt, tag + " y")
        same(x.grad, dXo if gi else dXt, tag + " dX")
        same(lin.weight.grad, dWo if gw else dWt, tag + " dW")


def test_weight_gradient_only_and_sr_steps():
    M, K, N = 128, 256, 160
    X = gaussian_bf16(M, K, seed=21).cuda()
    W = gaussian_bf16(N, K, seed=22, std=0.02).cuda()
    G = gaussian_bf16(M, N, seed=23, std=1e-3).cuda()
    Xb, Wb, Gb = tensor_bits(X), tensor_bits(W), tensor_bits(G)
    lin = T.Int8MixedPrecisionLinear(K, N, T.Int8MixedPrecisionConfig(stochastic_rounding=True), seed=41).cuda()
    with torch.no_grad():
        lin.weight.copy_(W)
    y0 = lin(X)  # input without grad: only dW is computed
    y0.backward(G)
    same(y0, oracle.linear_fwd(Xb, Wb, oracle.SR, 41, 0), "step 0 y")
    same(lin.weight.grad, oracle.linear_bwd(Gb, Xb, Wb, oracle.SR, 41, 0, want_dx=False)[1], "step 0 dW")
    y1 = lin(X)
    same(y1, oracle.linear_fwd(Xb, Wb, oracle.SR, 41, T.STEP_STRIDE), "step 1 y")
    assert not torch.equal(y0, y1)


def test_fp8_mlp_matches_fp8_chains():
    """The FP8 switch: the MLP's output and gradients equal the library's FP8
    chains run directly (whose parity with the oracle is in test_gpu_fp8.py)."""
    B, S, K1, H, N = 2, 64, 256, 512, 192
    x = gaussian_bf16(B * S, K1, seed=31).view(B, S, K1).cuda().requires_grad_()
    W1 = gaussian_bf16(H, K1, seed=32, std=0.02).cuda()
    W2 = gaussian_bf16(N, H, seed=33, std=0.02).cuda()
    G = gaussian_bf16(B * S, N, seed=34, std=1e-3).view(B, S, N).cuda()
    model = torch.nn.Sequential(torch.nn.Linear(K1, H, bias=False), torch.nn.ReLU(),
                                torch.nn.Linear(H, N, bias=False)).to(torch.bfloat16).cuda()
    with torch.no_grad():
        model[0].weight.copy_(W1)
        model[2].weight.copy_(W2)
    T.swap_linear_modules(model, T.Int8MixedPrecisionConfig(fp8=True))
    y = model(x)
    y.backward(G)
    X2 = x.detach().view(-1, K1)
    Y1 = i8.linear_fwd_fp8(X2, W1)
    Hh = torch.relu(Y1)
    Y2 = i8.linear_fwd_fp8(Hh, W2)
    dH, dW2 = i8.linear_bwd_fp8(G.view(-1, N), Hh, W2)
    dY1 = torch.where(Y1 > 0, dH, torch.zeros_like(dH))
    dX, dW1 = i8.linear_bwd_fp8(dY1, X2, W1)
    for got, want, what in ((y.view(-1, N), Y2, "y"), (x.grad.view(-1, K1), dX, "dX"),
                            (model[0].weight.grad, dW1, "dW1"), (model[2].weight.grad, dW2, "dW2")):
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), what


def _sr_mlp(seed_cfg=17):
    K1, H, N = 256, 512, 192
    W1 = gaussian_bf16(H, K1, seed=41, std=0.02).cuda()
    W2 = gaussian_bf16(N, H, seed=42, std=0.02).cuda()
    m = torch.nn.Sequential(torch.nn.Linear(K1, H, bias=False), torch.nn.ReLU(),
                            torch.nn.Linear(H, N, bias=False)).to(torch.bfloat16).cuda()
    with torch.no_grad():
        m[0].weight.copy_(W1)
        m[2].weight.copy_(W2)
    return T.swap_linear_modules(m, T.Int8MixedPrecisionConfig(stochastic_rounding=True, seed=seed_cfg))


def _sr_step(m, ckpt=None):
    """One forward + backward; ckpt: None (no checkpointing), "bare"
    (checkpointing without the contexts) or "replay" (with them)."""
    from torch.utils.checkpoint import checkpoint
    x = gaussian_bf16(128, 256, seed=43).cuda().requires_grad_()
    G = gaussian_bf16(128, 192, seed=44, std=1e-3).cuda()
    for p in m.parameters():
        p.grad = None
    if ckpt is None:
        y = m(x)
    elif ckpt == "bare":
        y = checkpoint(m, x, use_reentrant=False)
    else:
        y = checkpoint(m, x, use_reentrant=False, context_fn=T.sr_checkpoint_contexts)
    y.backward(G)
    return [t.detach().clone() for t in (y, x.grad, m[0].weight.grad, m[2].weight.grad)]


def _same_all(a, b):
    return all(torch.equal(u.view(torch.int16), v.view(torch.int16)) for u, v in zip(a, b))


def test_resumed_sr_run_equals_uninterrupted_run():
    """Stochastic rounding: a model whose state dict (seed and step of every
    swapped linear) is saved after two steps and loaded into a fresh model
    (built with another seed) draws in its third step exactly what the
    uninterrupted model draws: output and all gradients byte-identical."""
    import io
    a = _sr_mlp()
    steps = [_sr_step(a) for _ in range(3)]
    assert not _same_all(steps[0], steps[2])  # the step's draws matter
    b = _sr_mlp()
    _sr_step(b), _sr_step(b)
    buf = io.BytesIO()
    torch.save(b.state_dict(), buf)
    buf.seek(0)
    c = _sr_mlp(seed_cfg=12345)
    c.load_state_dict(torch.load(buf, weights_only=True))
    assert _same_all(_sr_step(c), steps[2])


def test_checkpointed_sr_step_equals_plain_step():
    """Activation checkpointing with sr_checkpoint_contexts: the recomputed
    forward replays the original draws, so output and gradients equal the
    run without checkpointing, step after step (and a recompute that drew
    anew, without the contexts, would not)."""
    a, b, c = _sr_mlp(), _sr_mlp(), _sr_mlp()
    for _ in range(2):
        plain = _sr_step(a)
        assert _same_all(_sr_step(b, "replay"), plain)
    assert not _same_all(_sr_step(c, "bare"), _sr_step(_sr_mlp()))
