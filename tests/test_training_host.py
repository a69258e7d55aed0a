"""Host-side logic of the training integration (no GPU): which modules are
swapped, that weights are shared, per-module seeds, the Philox offset a layer
hands to each step, and argument checks that fail before any device work."""
import pytest
import torch

i8 = pytest.importorskip("int8_mixed_precision_rowwise_amd")
from int8_mixed_precision_rowwise_amd import training as T  # noqa: E402


def model():
    return torch.nn.Sequential(
        torch.nn.Linear(8, 16, bias=False),
        torch.nn.ReLU(),
        torch.nn.Sequential(torch.nn.Linear(16, 4, bias=False)),
        torch.nn.Linear(4, 2, bias=True),
    ).to(torch.bfloat16)


def test_swap_replaces_bias_free_linears_and_shares_weights():
    m = model()
    w0, w2, w3 = m[0].weight, m[2][0].weight, m[3].weight
    T.swap_linear_modules(m, T.Int8MixedPrecisionConfig(seed=5))
    assert isinstance(m[0], T.Int8MixedPrecisionLinear)
    assert isinstance(m[2][0], T.Int8MixedPrecisionLinear)
    assert type(m[3]) is torch.nn.Linear  # has a bias: untouched
    assert m[0].weight is w0 and m[2][0].weight is w2 and m[3].weight is w3
    assert m[0].seed == T.module_seed(5, 0) and m[2][0].seed == T.module_seed(5, 1)
    assert m[0].seed != m[2][0].seed
    names = [n for n, _ in m.named_parameters()]
    assert names == ["0.weight", "2.0.weight", "3.weight", "3.bias"]


def test_swap_filter_and_root():
    m = model()
    T.swap_linear_modules(m, filter_fn=lambda mod, name: name.startswith("2"))
    assert type(m[0]) is torch.nn.Linear and isinstance(m[2][0], T.Int8MixedPrecisionLinear)
    bare = torch.nn.Linear(4, 4, bias=False)
    assert T.swap_linear_modules(bare) is bare and type(bare) is torch.nn.Linear
    with pytest.raises(ValueError):
        T.Int8MixedPrecisionLinear.from_linear(torch.nn.Linear(2, 2), T.Int8MixedPrecisionConfig(), 0)


def test_module_seed_values():
    seeds = {T.module_seed(0, i) for i in range(1000)} | {T.module_seed(1, i) for i in range(1000)}
    assert len(seeds) == 2000 and all(0 <= s < 2**64 for s in seeds)


def test_offsets_advance_per_training_step(monkeypatch):
    calls = []

    def fake_apply(x, w, cfg, seed, offset):
        calls.append((seed, offset))
        return x

    monkeypatch.setattr(T.Int8MixedPrecisionLinearFunction, "apply", staticmethod(fake_apply))
    lin = T.Int8MixedPrecisionLinear(4, 4, T.Int8MixedPrecisionConfig(stochastic_rounding=True), seed=9)
    x = torch.zeros(2, 4, dtype=torch.bfloat16)
    lin(x), lin(x)
    lin.eval()
    lin(x), lin(x)
    assert calls == [(9, 0), (9, T.STEP_STRIDE), (9, 2 * T.STEP_STRIDE), (9, 2 * T.STEP_STRIDE)]
    # a step's six quantize passes (offset + j * 2**40, j < 6) stay below the next step's offset
    assert 6 * (1 << 40) <= T.STEP_STRIDE


def test_config_and_argument_checks():
    c = T.Int8MixedPrecisionConfig()
    assert (c.output, c.grad_input, c.grad_weight, c.rounding) == (True, True, True, "rne")
    assert T.Int8MixedPrecisionConfig(stochastic_rounding=True).rounding == "sr"
    with pytest.raises(TypeError):
        T.Int8MixedPrecisionLinearFunction.apply(torch.zeros(2, 4), torch.zeros(3, 4), c, 0, 0)
    with pytest.raises(ValueError):
        T.Int8MixedPrecisionLinearFunction.apply(torch.zeros(2, 4, dtype=torch.bfloat16),
                                                 torch.zeros(3, 5, dtype=torch.bfloat16), c, 0, 0)
    assert "grad_weight=int8" in repr(T.Int8MixedPrecisionLinear(4, 4))


def test_fp8_config():
    c = T.Int8MixedPrecisionConfig(fp8=True)
    assert c.fp8 and c.rounding == "rne"
    with pytest.raises(ValueError):
        T.Int8MixedPrecisionConfig(fp8=True, stochastic_rounding=True)
    assert "codes=fp8_e4m3" in repr(T.Int8MixedPrecisionLinear(4, 4, c))


def test_key_rotates_when_the_offsets_run_out():
    assert T.STEPS_PER_KEY * T.STEP_STRIDE == 2**64
    last = T.STEPS_PER_KEY - 1
    assert T.step_key_offset(9, last) == (9, last * T.STEP_STRIDE)
    assert T.step_key_offset(9, T.STEPS_PER_KEY) == (T.module_seed(9, 1), 0)
    assert T.step_key_offset(9, 2 * T.STEPS_PER_KEY + 3) == (T.module_seed(9, 2), 3 * T.STEP_STRIDE)
    with pytest.raises(ValueError):
        T.step_key_offset(9, -1)


def _recording(monkeypatch):
    calls = []

    def fake_apply(x, w, cfg, seed, offset):
        calls.append((seed, offset))
        return x @ w.t()

    monkeypatch.setattr(T.Int8MixedPrecisionLinearFunction, "apply", staticmethod(fake_apply))
    return calls


def test_sr_state_is_in_the_state_dict(monkeypatch, tmp_path):
    """seed and step travel with the state dict (also through torch.save and
    a weights-only load), so a resumed module continues the stream."""
    calls = _recording(monkeypatch)
    cfg = T.Int8MixedPrecisionConfig(stochastic_rounding=True, seed=3)
    m = T.swap_linear_modules(torch.nn.Sequential(torch.nn.Linear(4, 4, bias=False)).to(torch.bfloat16), cfg)
    x = torch.zeros(2, 4, dtype=torch.bfloat16)
    for _ in range(3):
        m(x)
    sd = m.state_dict()
    assert sd["0._extra_state"] == {"seed": T.module_seed(3, 0), "step": 3}
    path = tmp_path / "ckpt.pt"
    torch.save(sd, path)
    fresh = T.swap_linear_modules(torch.nn.Sequential(torch.nn.Linear(4, 4, bias=False)).to(torch.bfloat16),
                                  T.Int8MixedPrecisionConfig(stochastic_rounding=True, seed=99))
    fresh.load_state_dict(torch.load(path, weights_only=True))
    assert (fresh[0].seed, fresh[0].step) == (m[0].seed, 3)
    calls.clear()
    m(x), fresh(x)
    assert calls[0] == calls[1] == (T.module_seed(3, 0), 3 * T.STEP_STRIDE)
    with pytest.raises(ValueError):
        fresh[0].set_extra_state({"seed": -1, "step": 0})


def test_checkpoint_recompute_replays_the_forward_draws(monkeypatch):
    """Under torch.utils.checkpoint with sr_checkpoint_contexts, the
    recomputed forward uses the original (key, offset) of every layer and the
    step advances once per training forward, as without checkpointing."""
    from torch.utils.checkpoint import checkpoint
    calls = _recording(monkeypatch)
    cfg = T.Int8MixedPrecisionConfig(stochastic_rounding=True, seed=5)
    m = T.swap_linear_modules(torch.nn.Sequential(torch.nn.Linear(4, 8, bias=False), torch.nn.ReLU(),
                                                  torch.nn.Linear(8, 4, bias=False)).to(torch.bfloat16), cfg)
    x = torch.randn(3, 4, dtype=torch.bfloat16, requires_grad=True)
    for step in range(2):
        calls.clear()
        y = checkpoint(m, x, use_reentrant=False, context_fn=T.sr_checkpoint_contexts)
        y.float().sum().backward()
        k0, k2 = T.module_seed(5, 0), T.module_seed(5, 1)
        first = [(k0, step * T.STEP_STRIDE), (k2, step * T.STEP_STRIDE)]
        assert calls == first + first  # forward, then the recompute with the same draws
        assert m[0].step == m[2].step == step + 1
    assert T._ckpt.mode is None and T._ckpt.log is None
