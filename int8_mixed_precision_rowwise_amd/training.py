"""Training integration: an autograd op and a module swap over the C ABI.

This is the user boundary the pages describe, restated for this library:
- weights of bias-free ``nn.Linear`` modules are swapped so that each linear's
  forward and its two backward GEMMs run as INT8 mixed precision ("Integrate
  INT8 mixed-precision from torchao 0.7", the usage reply: ``quantize_`` with a
  filter over modules);
- each of the three GEMMs can be INT8 or BF16 on its own, and stochastic
  rounding can be switched on ("Quantized model training", section "INT8 mixed
  precision training", the ablation table: forward, backward grad input,
  backward grad weight, stochastic rounding).

Every INT8 GEMM and its quantization passes run in ``libi8mp``'s kernels
(``linear_fwd`` / ``linear_bwd``).  A GEMM switched to BF16 is a plain bf16
matmul by torch (hipBLASLt): that is the configuration's meaning, not a
fallback.  Inputs, weights and gradients are bf16.  With ``fp8`` set, the
quantized GEMMs take the row-wise FP8 (E4M3) path instead (``linear_fwd_fp8``
/ ``linear_bwd_fp8``; round to nearest), the row-wise FP8 recipe that
"Quantized model training" sets beside INT8 mixed precision.

Stochastic rounding draws from Philox4x32-10 keyed by a per-module seed; the
layer's step counter advances the counter offset by ``STEP_STRIDE`` per forward
call, so every quantize pass of every step draws fresh numbers and a run is
reproducible from the seed.  The backward of a step reuses its forward's
(seed, offset): the six quantize passes of one step use offsets
``offset + j * 2**40``, j = 0..5.  The 64-bit offset holds ``STEPS_PER_KEY``
steps; past that the key moves on (``step_key_offset``), so draws never repeat.

The seed and the step counter are part of the module's state dict (its extra
state), so a run resumed from a checkpoint continues the same stream.  Under
activation checkpointing (``torch.utils.checkpoint.checkpoint`` with
``use_reentrant=False`` and ``context_fn=sr_checkpoint_contexts``) the
recomputed forward replays the (key, offset) of the original forward instead
of drawing new numbers, so its activations and the gradients equal those of a
run without checkpointing.
"""
from __future__ import annotations

import dataclasses
import threading
from typing import Callable, Optional

import torch

from . import linear_bwd, linear_bwd_fp8, linear_fwd, linear_fwd_colmax, linear_fwd_fp8, linear_fwd_fp8_colmax

__all__ = ["Int8MixedPrecisionConfig", "Int8MixedPrecisionLinearFunction",
           "Int8MixedPrecisionLinear", "swap_linear_modules", "STEP_STRIDE", "STEPS_PER_KEY",
           "module_seed", "step_key_offset", "sr_checkpoint_contexts"]

STEP_STRIDE = 8 << 40  # Philox blocks reserved per linear step (6 passes of 2**40 each, rounded up)
STEPS_PER_KEY = (1 << 64) // STEP_STRIDE  # steps whose offsets fit the 64-bit block counter


@dataclasses.dataclass(frozen=True)
class Int8MixedPrecisionConfig:
    """Which GEMMs of a linear layer run in INT8, and how codes are rounded.

    output: forward Y = X @ W.T; grad_input: dX = dY @ W; grad_weight:
    dW = dY.T @ X.  A GEMM left False runs as a bf16 matmul.  fp8: the
    quantized GEMMs use FP8 (E4M3) codes and the FP8 matrix core instead of
    INT8 (round to nearest only; every quantized GEMM's contraction length a
    multiple of 16 and its output extents along operands read down their
    rows multiples of 4).
    """
    output: bool = True
    grad_input: bool = True
    grad_weight: bool = True
    stochastic_rounding: bool = False
    seed: int = 0
    fp8: bool = False

    def __post_init__(self):
        if self.fp8 and self.stochastic_rounding:
            raise ValueError("the FP8 variant rounds to nearest only")

    @property
    def rounding(self) -> str:
        return "sr" if self.stochastic_rounding else "rne"


def module_seed(base_seed: int, index: int) -> int:
    """Philox key of the index-th swapped module: a SplitMix64 step of
    (base_seed + index), so neighbouring modules get unrelated keys."""
    z = (base_seed + (index + 1) * 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
    return z ^ (z >> 31)


def step_key_offset(seed: int, step: int) -> tuple[int, int]:
    """(Philox key, counter offset) of a module's step-th training forward.
    Steps 0 .. STEPS_PER_KEY-1 use the module's seed with offset
    step * STEP_STRIDE; each later run of STEPS_PER_KEY steps uses the key
    module_seed(seed, step // STEPS_PER_KEY) (a SplitMix64 step away from the
    seed) with the offsets starting again at 0, so no (key, offset) pair of a
    module repeats."""
    if step < 0:
        raise ValueError(f"step must be >= 0, got {step}")
    epoch, within = divmod(step, STEPS_PER_KEY)
    key = seed if epoch == 0 else module_seed(seed, epoch)
    return key, within * STEP_STRIDE


class _CheckpointState(threading.local):
    mode: Optional[str] = None  # None, "record" (original forward) or "replay" (recompute)
    log: Optional[list] = None


_ckpt = _CheckpointState()


class _SrContext:
    """Enters one of the two modes of a checkpointed region (see
    sr_checkpoint_contexts); the previous mode comes back on exit."""

    def __init__(self, mode: str, log: list):
        self.mode, self.log = mode, log

    def __enter__(self):
        self.saved = (_ckpt.mode, _ckpt.log)
        _ckpt.mode, _ckpt.log = self.mode, self.log
        return self

    def __exit__(self, *exc):
        _ckpt.mode, _ckpt.log = self.saved
        return False


def sr_checkpoint_contexts():
    """Context managers for ``torch.utils.checkpoint.checkpoint(fn, *args,
    use_reentrant=False, context_fn=sr_checkpoint_contexts)``: during the
    original forward every INT8 mixed-precision linear of the region records
    the (key, offset) it drew with; during the recompute it replays them in
    the same order instead of advancing its step.  One checkpointed region at
    a time (no nesting)."""
    log: list = []
    return _SrContext("record", log), _SrContext("replay", log)


def _as_rows(t: torch.Tensor, cols: int) -> torch.Tensor:
    t2 = t.reshape(-1, cols)
    return t2 if t2.is_contiguous() else t2.contiguous()


class Int8MixedPrecisionLinearFunction(torch.autograd.Function):
    """y = x @ weight.T (bias-free), x [..., K], weight [N, K], all bf16.

    Saved for backward: the bf16 input and weight (what the pages' op keeps;
    nothing quantized is stored), plus, when the forward GEMM is INT8, the
    column maxima of both (fp32, K values each) that its row-wise passes
    produce and the backward's column-wise passes need."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, weight: torch.Tensor, config: Int8MixedPrecisionConfig,
                seed: int, offset: int):
        if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
            raise TypeError("INT8 mixed-precision linear takes bf16 input and weight, got "
                            f"{x.dtype} and {weight.dtype}")
        if weight.dim() != 2 or x.shape[-1] != weight.shape[1]:
            raise ValueError(f"shapes {tuple(x.shape)} and {tuple(weight.shape)} do not match")
        lead = x.shape[:-1]
        x2 = _as_rows(x, x.shape[-1])
        w = weight if weight.is_contiguous() else weight.contiguous()
        cx = cw = None
        if config.output and config.fp8 and (config.grad_input or config.grad_weight):
            y, cx, cw = linear_fwd_fp8_colmax(x2, w)
        elif config.output and config.fp8:
            y = linear_fwd_fp8(x2, w)
        elif config.output and (config.grad_input or config.grad_weight):
            y, cx, cw = linear_fwd_colmax(x2, w, config.rounding, seed, offset)
        elif config.output:
            y = linear_fwd(x2, w, config.rounding, seed, offset)
        else:
            y = torch.mm(x2, w.t())
        ctx.save_for_backward(x2, w, cx, cw)
        ctx.config, ctx.seed, ctx.offset, ctx.lead = config, seed, offset, lead
        return y.view(*lead, w.shape[0])

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x2, w, cx, cw = ctx.saved_tensors
        cfg = ctx.config
        need_dx, need_dw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        dy2 = _as_rows(dy.to(torch.bfloat16), w.shape[0])
        int_dx, int_dw = need_dx and cfg.grad_input, need_dw and cfg.grad_weight
        dx = dw = None
        if (int_dx or int_dw) and cfg.fp8:
            dx, dw = linear_bwd_fp8(dy2, x2, w, want_dx=int_dx, want_dw=int_dw, colmax_x=cx, colmax_w=cw)
        elif int_dx or int_dw:
            dx, dw = linear_bwd(dy2, x2, w, cfg.rounding, ctx.seed, ctx.offset,
                                want_dx=int_dx, want_dw=int_dw, colmax_x=cx, colmax_w=cw)
        if need_dx and not int_dx:
            dx = torch.mm(dy2, w)
        if need_dw and not int_dw:
            dw = torch.mm(dy2.t(), x2)
        if dx is not None:
            dx = dx.view(*ctx.lead, w.shape[1])
        return dx, dw, None, None, None


class Int8MixedPrecisionLinear(torch.nn.Linear):
    """Bias-free linear layer whose GEMMs run per ``config``.

    ``seed`` keys this module's stochastic-rounding stream; ``step`` counts its
    training forward calls (step_key_offset gives the Philox key and offset of
    a call).  Both are saved in the state dict as the module's extra state and
    restored by load_state_dict, so a resumed run draws what an uninterrupted
    one would."""

    def __init__(self, in_features: int, out_features: int,
                 config: Optional[Int8MixedPrecisionConfig] = None, seed: int = 0,
                 device=None, dtype=torch.bfloat16):
        super().__init__(in_features, out_features, bias=False, device=device, dtype=dtype)
        self.config = config or Int8MixedPrecisionConfig()
        self.seed = seed
        self.step = 0

    @classmethod
    def from_linear(cls, lin: torch.nn.Linear, config: Int8MixedPrecisionConfig,
                    seed: int) -> "Int8MixedPrecisionLinear":
        """Wrap an existing bias-free linear, keeping its weight Parameter (same
        object, so optimizers and state dicts see no change)."""
        if lin.bias is not None:
            raise ValueError("INT8 mixed-precision linear layers are bias-free")
        new = cls.__new__(cls)
        torch.nn.Module.__init__(new)
        new.in_features, new.out_features = lin.in_features, lin.out_features
        new.weight = lin.weight
        new.register_parameter("bias", None)
        new.config, new.seed, new.step = config, seed, 0
        return new

    def get_extra_state(self):
        return {"seed": int(self.seed), "step": int(self.step)}

    def set_extra_state(self, state):
        if not isinstance(state, dict) or set(state) != {"seed", "step"}:
            raise ValueError(f"expected {{'seed', 'step'}} extra state, got {state!r}")
        seed, step = int(state["seed"]), int(state["step"])
        if not (0 <= seed < 2**64 and step >= 0):
            raise ValueError(f"seed must be in [0, 2**64) and step >= 0, got {seed}, {step}")
        self.seed, self.step = seed, step

    def _key_offset(self) -> tuple[int, int]:
        """(key, offset) of this call; a training call outside a replay
        advances the step."""
        if _ckpt.mode == "replay" and self.training:
            if not _ckpt.log or _ckpt.log[0][0] is not self:
                raise RuntimeError("checkpoint recompute reached an INT8 mixed-precision linear "
                                   "that the original forward did not (or in another order)")
            return _ckpt.log.pop(0)[1]
        ko = step_key_offset(self.seed, self.step)
        if self.training:
            self.step += 1
            if _ckpt.mode == "record":
                _ckpt.log.append((self, ko))
        return ko

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        key, offset = self._key_offset()
        return Int8MixedPrecisionLinearFunction.apply(x, self.weight, self.config, key, offset)

    def extra_repr(self) -> str:
        c = self.config
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"output={'int8' if c.output else 'bf16'}, grad_input={'int8' if c.grad_input else 'bf16'}, "
                f"grad_weight={'int8' if c.grad_weight else 'bf16'}, rounding={c.rounding}"
                + (", codes=fp8_e4m3" if c.fp8 else ""))


def swap_linear_modules(model: torch.nn.Module, config: Optional[Int8MixedPrecisionConfig] = None,
                        filter_fn: Optional[Callable[[torch.nn.Module, str], bool]] = None
                        ) -> torch.nn.Module:
    """Replace, in place, every bias-free ``nn.Linear`` of ``model`` for which
    ``filter_fn(module, qualified_name)`` holds (all of them by default) with an
    ``Int8MixedPrecisionLinear`` that shares its weight.  Linears with a bias
    are left alone.  Modules are numbered in ``named_modules`` order; the n-th
    swapped module's seed is ``module_seed(config.seed, n)``.  Returns model."""
    config = config or Int8MixedPrecisionConfig()
    targets = []
    for name, mod in model.named_modules():
        if not name:
            continue  # the root module is not replaced (wrap a bare Linear in a container)
        if type(mod) is torch.nn.Linear and mod.bias is None and (filter_fn is None or filter_fn(mod, name)):
            targets.append(name)
    for index, name in enumerate(targets):
        parent_name, _, child = name.rpartition(".")
        parent = model.get_submodule(parent_name) if parent_name else model
        lin = getattr(parent, child)
        setattr(parent, child, Int8MixedPrecisionLinear.from_linear(lin, config, module_seed(config.seed, index)))
    return model
