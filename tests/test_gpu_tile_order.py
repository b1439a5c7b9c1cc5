"""Tile launches that take tiles biggest first (the tile order written by
route preparation) against tiles in route order: the same bits, on
NaN-poisoned workspaces and outputs (a tile missing from the order would
leave its rows poisoned, a tile listed twice would leave another one out),
over tile-size mixes from full 64-row tiles to one-subtile tails, a skewed
routing with many tiles per hot expert, both down kernels, the opted-in fp16
route and the fused finalize."""
import numpy as np
import pytest
import torch

from moe_check import assert_close, bits, oracle_out, tokens, weights
from w4a16_mixture_experts_amd import binding, synth

pytestmark = pytest.mark.gpu


def _run(wl, Wg, tg, T, **force):
    d = binding.desc_for(wl, T, force_path=1, **force)
    ws = torch.full((binding.workspace_size(d),), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.full((T, wl.hidden), float("nan"), dtype=wl.dtype, device="cuda")
    binding.forward_workload(wl, Wg, tg, out=out, workspace=ws, force_path=1, **force)
    torch.cuda.synchronize()
    return out


CASES = [("tiny", 256, {}), ("tiny", 100, {}), ("tiny", 600, {}), ("tiny", 256, {"fp16_route": 1}),
         ("tiny", 256, {"fused_finalize": 1}), ("relu2_skew", 1024, {}),
         ("deepseek_local", 512, {}), ("per_channel", 256, {}), ("kimi_tp8", 2048, {}),
         ("kimi_tp8", 1024, {"fused_finalize": 1})]


@pytest.mark.parametrize("name,T,extra", CASES,
                         ids=[f"{n}-{t}-{'-'.join(f'{k}{v}' for k, v in e.items())}" for n, t, e in CASES])
def test_tile_order_same_bits(name, T, extra):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    assert binding.get_plan(binding.desc_for(wl, T, force_path=1, force_tile_order=2,
                                             **extra)).tile_order == 1
    assert binding.get_plan(binding.desc_for(wl, T, force_path=1, force_tile_order=1,
                                             **extra)).tile_order == 0
    tc = tokens(wl, T)
    tg = tc.to("cuda")
    a = _run(wl, Wg, tg, T, force_tile_order=1, **extra)
    b = _run(wl, Wg, tg, T, force_tile_order=2, **extra)
    assert not torch.isnan(b.float()).any()
    np.testing.assert_array_equal(bits(a), bits(b))
    if wl.num_experts * wl.hidden * wl.n1 <= 5e7:   # small shapes: the whole output
        assert_close(b, oracle_out(wl, Wc, tc), f"{name} T={T} biggest tiles first")
