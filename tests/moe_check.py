"""Shared helpers of the GPU parity tests: input caching, the oracle call and
the tolerance checks (NRMSE <= 5e-3 and max-abs <= 2e-2 against the FP32
oracle, as the spec bar states)."""
import functools
import sys

import numpy as np
import torch

import oracle
from w4a16_mixture_experts_amd import binding, synth

NRMSE_TOL = 5e-3
MAXABS_TOL = 2e-2


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@functools.lru_cache(maxsize=4)
def weights(name: str):
    """(cpu Weights, gpu Weights) of a named workload; big ones are drawn on the GPU."""
    wl = synth.WORKLOADS[name]
    big = wl.num_experts * wl.hidden * wl.n1 > 5e7
    dev = "cuda" if big else "cpu"
    W = synth.make_weights(wl, device=dev)
    return W.to("cpu"), W.to("cuda")


def tokens(wl, T: int, device="cpu"):
    tok = synth.make_tokens(wl, T, device="cpu")
    return tok if device == "cpu" else tok.to(device)


def oracle_out(wl, Wc, tok_cpu, rows=None):
    """FP32 oracle output for all tokens, or for the token rows listed."""
    x, ids, w = tok_cpu.x, tok_cpu.topk_ids, tok_cpu.topk_weights
    if rows is not None:
        idx = torch.as_tensor(rows)
        x, ids, w = x[idx], ids[idx], w[idx]
    return oracle.moe_forward(
        bits(x), Wc.w13_packed.numpy(), bits(Wc.w13_scales), Wc.w2_packed.numpy(),
        bits(Wc.w2_scales), ids.numpy(), w.numpy(), hidden=wl.hidden, inter=wl.inter,
        num_experts=wl.num_experts, expert_offset=wl.expert_offset,
        act=oracle.ACT_SILU_GATED if wl.gated else oracle.ACT_RELU2,
        layout=(oracle.Q_PER_CHANNEL if wl.per_channel
                else oracle.Q_FP4_GROUP_K if wl.fp4 else oracle.Q_GROUP_K),
        dtype=oracle.DT_FP16 if wl.dtype == torch.float16 else oracle.DT_BF16)


def errors(gpu: torch.Tensor, ref: np.ndarray):
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    r = ref.astype(np.float64)
    assert g.shape == r.shape
    assert np.isfinite(g).all(), "non-finite GPU output"
    nr = np.linalg.norm(r)
    diff = g - r
    nrmse = np.linalg.norm(diff) / nr if nr > 0 else (0.0 if not diff.any() else np.inf)
    return float(nrmse), float(np.abs(diff).max(initial=0.0))


def row_errors(gpu: torch.Tensor, ref: np.ndarray) -> np.ndarray:
    """NRMSE of every token row (the same definition over one row's H
    outputs); a row whose oracle output is all zeros gets 0 if the GPU row is
    exactly zero too, else inf."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64).reshape(ref.shape[0], -1)
    r = ref.astype(np.float64).reshape(ref.shape[0], -1)
    nr = np.linalg.norm(r, axis=1)
    nd = np.linalg.norm(g - r, axis=1)
    out = np.where(nr > 0, nd / np.where(nr > 0, nr, 1.0), np.where(nd > 0, np.inf, 0.0))
    return out


def assert_close(gpu, ref, what=""):
    """Whole-output NRMSE and max-abs against the bar, and the same NRMSE
    bar for every token row on its own (one wrong row cannot hide in the
    average)."""
    nrmse, maxabs = errors(gpu, ref)
    rows = row_errors(gpu, ref) if ref.ndim == 2 and ref.shape[0] > 0 else np.zeros(0)
    worst = float(rows.max(initial=0.0))
    sys.__stderr__.write(f"[parity] {what} nrmse={nrmse:.3e} maxabs={maxabs:.3e} "
                         f"worst_row_nrmse={worst:.3e}\n")
    sys.__stderr__.flush()
    assert nrmse <= NRMSE_TOL, f"{what}: NRMSE {nrmse:.3e} > {NRMSE_TOL}"
    assert maxabs <= MAXABS_TOL, f"{what}: max-abs {maxabs:.3e} > {MAXABS_TOL}"
    bad = np.nonzero(rows > NRMSE_TOL)[0]
    assert bad.size == 0, f"{what}: rows {bad[:8].tolist()} NRMSE {rows[bad[:8]].tolist()}"
    return nrmse, maxabs


def forward(wl, Wg, tok_gpu, **kw):
    out = binding.forward_workload(wl, Wg, tok_gpu, **kw)
    torch.cuda.synchronize()
    return out
