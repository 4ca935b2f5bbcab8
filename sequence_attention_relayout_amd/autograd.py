"""Differentiable Ulysses relayout for PyTorch (a torch.autograd.Function).

The relayout is a permutation of elements, so its adjoint is its inverse:
the backward of mode 0 is mode 1 with the same plan, and the backward of
mode 1 is mode 0 (fast-ulysses 0.2.1 README, "Quick start" and "Limits":
the collective is differentiable; FastVideo "Ulysses performance on GB200":
backward uses the plan saved by its forward).  Both directions run in
libulysses.so; torch only allocates the outputs and gradients.
"""
import torch

from . import ulysses as U

__all__ = ["all_to_all_4d"]


def _empty_outputs(plan, mode, like):
    return [torch.empty(U.ulysses_plan_shape(plan, mode, r, True), dtype=like.dtype,
                        device=like.device) for r in range(plan.world)]


class _AllToAll4D(torch.autograd.Function):
    @staticmethod
    def forward(ctx, plan, mode, *xs):
        xs = [x.contiguous() for x in xs]
        outs = _empty_outputs(plan, mode, xs[0])
        U.ulysses_a2a_4d(plan, mode, xs, outs)
        ctx.plan, ctx.mode = plan, mode
        return tuple(outs)

    @staticmethod
    def backward(ctx, *grads):
        plan, inv = ctx.plan, 1 - ctx.mode
        # a destination shard that received no gradient contributes zeros
        ref = next(g for g in grads if g is not None)
        gs = [g.contiguous() if g is not None else
              torch.zeros(U.ulysses_plan_shape(plan, inv, r, False), dtype=ref.dtype,
                          device=ref.device) for r, g in enumerate(grads)]
        outs = _empty_outputs(plan, inv, gs[0])
        U.ulysses_a2a_4d(plan, inv, gs, outs)
        return (None, None, *outs)


def all_to_all_4d(plan, xs, mode=0):
    """The relayout of the W shards `xs` (torch tensors on the GPU, the
    plan's dtype and input shapes for `mode`); returns the W output shards,
    differentiable with respect to the inputs."""
    if len(xs) != plan.world:
        raise ValueError(f"need {plan.world} shards, got {len(xs)}")
    esz = U.ELEM_BYTES[plan.dtype]
    for r, x in enumerate(xs):
        if x.element_size() != esz:
            raise ValueError(f"shard {r}: {x.dtype} does not have the plan's {esz}-byte elements")
        if tuple(x.shape) != U.ulysses_plan_shape(plan, mode, r, False):
            raise ValueError(f"shard {r}: shape {tuple(x.shape)}, the plan's is "
                             f"{U.ulysses_plan_shape(plan, mode, r, False)}")
    return list(_AllToAll4D.apply(plan, int(mode), *xs))
