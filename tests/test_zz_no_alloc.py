"""The no-alloc forward (w4a16_moe_forward_noalloc, scratch in a library-owned
device array) against the workspace forward on the same inputs: identical
bits, on two calls in a row whose second input is smaller (the array keeps the
first call's contents), and within the oracle's tolerance."""
import pytest
import torch

from moe_check import assert_close, oracle_out, tokens, weights
from w4a16_mixture_experts_amd import binding, synth

pytestmark = pytest.mark.gpu


def _pair(wl, Wg, tg, **force):
    ref = binding.forward_workload(wl, Wg, tg, **force)
    out = torch.full((tg.x.shape[0], wl.hidden), float("nan"), dtype=wl.dtype, device="cuda")
    binding.forward_workload(wl, Wg, tg, out=out, no_alloc=True, **force)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("name,Ts,force", [
    ("kimi_tp8", (256, 32), {}),            # grouped streaming, then split-K
    ("kimi_tp8", (32, 8), {}),              # split-K, then the small-batch path
    ("tiny", (256, 16), dict(force_path=1)),
    ("relu2_skew", (1024, 32), {}),         # fp16, streaming down GEMM
    ("per_channel", (256, 8), {}),
])
def test_no_alloc_matches_workspace_forward(name, Ts, force):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    for T in Ts:
        d = binding.desc_for(wl, T, **force)
        assert binding.workspace_size(d) <= binding.NOALLOC_SCRATCH_BYTES
        tc = tokens(wl, T)
        out, ref = _pair(wl, Wg, tc.to("cuda"), **force)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (name, T)
        if T <= 256:
            assert_close(out, oracle_out(wl, Wc, tc), f"no-alloc {name} T={T}")


def test_no_alloc_rejects_oversized_workspace():
    wl = synth.WORKLOADS["kimi_tp8"]
    _, Wg = weights("kimi_tp8")
    T = 2048
    assert binding.workspace_size(binding.desc_for(wl, T)) > binding.NOALLOC_SCRATCH_BYTES
    tg = tokens(wl, T, "cuda")
    out = torch.empty(T, wl.hidden, dtype=wl.dtype, device="cuda")
    with pytest.raises(binding.W4A16Error) as ei:
        binding.forward_workload(wl, Wg, tg, out=out, no_alloc=True)
    assert ei.value.status == 2 and "no-alloc scratch" in ei.value.message
