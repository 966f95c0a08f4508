"""GPU: one work plan per decode iteration (pa_decode_plan with
pa_append_decode_planned / pa_decode_planned).

All layers of an iteration attend the same context lengths, so the plan a
split launch runs from can be made once and used by every layer.  The
planned calls must give the outputs and cache bytes of pa_append_decode /
pa_decode bit for bit (each partition is computed on its own and merged in
partition order, whatever order the plan lists them in), and the oracle's
outputs within the decode tolerances.  Cases: the ragged mix at batch 64
(a plan-using launch) over three layers, fused and unfused, with the
library's and an explicit partition size; a launch that uses no plan.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W

from gpu_harness import Case, check_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.synchronize()


def _workspace(case: Case, pt: int) -> torch.Tensor:
    cfg = case.cfg
    need = case.pool.workspace_bytes(cfg.batch, cfg.num_q_heads, case.max_context, pt)
    return torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")


def _planned(case: Case, layer: int, ws: torch.Tensor, pt: int, append=None) -> torch.Tensor:
    case.pool.check_decode_args(case.tables_np, case.lens_np, case.max_context,
                                slots=append[2].cpu().numpy() if append is not None else None)
    out = case.pool.decode(layer, case.vals[layer][0], case.scale, case.tables, case.lens,
                           case.max_context, partition_tokens=pt, workspace=ws, append=append,
                           planned=True)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("pt", [0, 512])
def test_one_plan_serves_every_layer_fused(pt):
    cfg = W.get(3, batch=64)
    layers = (0, 1, 2)
    # zero-filled pools, so that rows nobody writes compare equal too
    plan = Case(cfg, layers=layers, step_append=False, fill=0.0)
    own = Case(cfg, layers=layers, step_append=False, fill=0.0)
    assert torch.equal(plan.step_slots, own.step_slots)
    ws = _workspace(plan, pt)
    assert plan.pool.decode_plan(plan.lens, cfg.num_q_heads, plan.max_context, ws, pt)
    for layer in layers:
        k, v = plan.step_kv(layer)
        got = _planned(plan, layer, ws, pt, append=(k, v, plan.step_slots))
        exp = own.decode(layer=layer, partition_tokens=pt, append=(k, v, own.step_slots))
        assert torch.equal(got, exp), layer
        check_rows(plan, got, range(cfg.batch), layer=layer)
    assert torch.equal(plan.pool.kv_cache, own.pool.kv_cache)


def test_one_plan_serves_every_layer_unfused():
    cfg = W.get(3, batch=64, kv_dtype="f32", head_dim=64)
    layers = (0, 1, 2)
    case = Case(cfg, layers=layers)
    ws = _workspace(case, 0)
    assert case.pool.decode_plan(case.lens, cfg.num_q_heads, case.max_context, ws)
    for layer in reversed(layers):
        got = _planned(case, layer, ws, 0)
        # pa_decode rewrites an equivalent plan in the same place
        exp = case.decode(layer=layer)
        assert torch.equal(got, exp), layer
        check_rows(case, got, range(cfg.batch), layer=layer)


def test_launch_without_a_plan_runs_as_the_plain_call():
    # 8 sequences of 1025 tokens: a split launch of a few hundred workgroups,
    # too few for a plan, so none is made and the planned call is the plain
    # one (partitions and merge included)
    cfg = W.get(2, batch=8, num_blocks=8 * 64 + 3)
    case = Case(cfg, step_append=False, fill=0.0)
    ws = _workspace(case, 0)
    assert not case.pool.decode_plan(case.lens, cfg.num_q_heads, case.max_context, ws)
    k, v = case.step_kv()
    ref = Case(cfg, step_append=False, fill=0.0)
    got = _planned(case, 0, ws, 0, append=(k, v, case.step_slots))
    exp = ref.decode(append=(k, v, ref.step_slots))
    assert torch.equal(got, exp)
    assert torch.equal(case.pool.kv_cache, ref.pool.kv_cache)
    check_rows(case, got, range(cfg.batch))
