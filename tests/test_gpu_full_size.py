"""GPU parity over every token count of the five workloads' sweeps, in the
launch configuration the benchmark times (automatic plan).  Token counts the
oracle finishes in seconds are compared whole (the smallest ones in
test_gpu_parity); larger ones on sampled token rows that the oracle
recomputes one by one: each token's output depends only on its own routes,
so those rows are exact references for the rows the GPU produced inside the
full batch.  Every compared row must meet the NRMSE bar on its own."""
import numpy as np
import pytest
import torch

from moe_check import assert_close, forward, oracle_out, tokens, weights
from w4a16_mixture_experts_amd import synth

pytestmark = pytest.mark.gpu

WHOLE = [("kimi_tp8", 256), ("deepseek_local", 128), ("deepseek_local", 512),
         ("per_channel", 256)]
SAMPLED = [("kimi_tp8", 1024), ("kimi_tp8", 2048), ("deepseek_local", 2048),
           ("relu2_skew", 1024), ("relu2_skew", 4096),
           # the interface's largest token count: 524,280 routes, about 8,600
           # expert tiles, route preparation over its full 32 chunks
           ("kimi_tp8", 65535)]
N_SAMPLED = 32


def test_sweeps_are_covered():
    """Every (workload, token count) of the sweeps is compared somewhere."""
    small = {("tiny", 16), ("kimi_tp8", 1), ("kimi_tp8", 8), ("kimi_tp8", 32),
             ("deepseek_local", 1), ("deepseek_local", 16), ("per_channel", 1),
             ("per_channel", 8), ("relu2_skew", 32)}
    covered = small | set(WHOLE) | set(SAMPLED)
    # the FP4-weight workloads' sweeps are compared in test_gpu_fp4
    fp4 = {(n, T) for n in ("kimi_tp8_fp4",) for T in (1, 8, 32, 256, 1024, 2048)} | {
        (n, T) for n in ("deepseek_local_fp4",) for T in (1, 16, 128, 512, 2048)}
    covered |= fp4
    for name, wl in synth.WORKLOADS.items():
        for T in wl.tokens:
            assert (name, T) in covered, (name, T)


@pytest.mark.parametrize("name,T", WHOLE)
def test_full_size_whole_output(name, T):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tc = tokens(wl, T)
    out = forward(wl, Wg, tc.to("cuda"))
    assert_close(out, oracle_out(wl, Wc, tc), f"{name} T={T} whole")


@pytest.mark.parametrize("name,T", SAMPLED)
def test_full_size_sampled_rows(name, T):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tc = tokens(wl, T)
    out = forward(wl, Wg, tc.to("cuda"))
    rng = np.random.default_rng(T)
    rows = sorted(set([0, T - 1] + rng.choice(T, size=N_SAMPLED - 2, replace=False).tolist()))
    ref = oracle_out(wl, Wc, tc, rows=rows)
    assert_close(out[torch.as_tensor(rows, device="cuda")], ref, f"{name} T={T} rows={rows}")
    assert torch.isfinite(out.float()).all()
