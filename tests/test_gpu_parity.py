"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer work (nibble unpacking, route tables) must match bit for bit; the
16-bit MoE outputs must be within NRMSE <= 5e-3 and max-abs <= 2e-2 of the
FP32 oracle.  Sizes are chosen so the oracle finishes in seconds while still
spanning several tiles, split-K partitions and ragged tails.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from moe_check import assert_close, bits, errors, forward, oracle_out, tokens, weights
from w4a16_mixture_experts_amd import binding, synth

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# integer work: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 3, 4, 5, 256, 257, 4099])
def test_unpack_bit_exact(n):
    rng = np.random.default_rng(n)
    b = np.concatenate([np.arange(256, dtype=np.uint8), rng.integers(0, 256, n, dtype=np.uint8)])
    b = b[:n] if n < 256 else b
    got = binding.unpack_int4(torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.unpack_int4(b))


ROUTE_CASES = [
    # T, K, E, E_global, offset, block_m
    (1, 8, 384, 384, 0, 16), (8, 8, 384, 384, 0, 16), (16, 2, 8, 8, 0, 16),
    (2048, 8, 384, 384, 0, 64), (4096, 6, 128, 128, 0, 64), (2048, 8, 32, 256, 0, 64),
    (8192, 8, 384, 384, 0, 64), (300, 8, 384, 384, 0, 64), (129, 8, 60, 60, 0, 32),
    (7, 3, 5, 9, 2, 4), (33, 4, 60, 60, 0, 32), (100, 8, 1024, 1024, 0, 1),
    (5, 2, 8, 8, 0, 256), (0, 4, 8, 8, 0, 16),
    # one workgroup with 2 route pieces per wave, and two launches above it
    (256, 8, 384, 384, 0, 64), (512, 8, 384, 384, 0, 64), (513, 8, 384, 384, 0, 64),
    (170, 12, 60, 64, 2, 128), (1000, 4, 1024, 1024, 0, 16),
]


@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "one-chunk"])
@pytest.mark.parametrize("T,K,E,Eg,off,bm", ROUTE_CASES)
def test_route_prep_bit_exact(T, K, E, Eg, off, bm, chunked):
    rng = np.random.default_rng(T + 7 * K + E)
    ids = rng.integers(-3, Eg + 3, size=(T, K)).astype(np.int32)
    if T > 4:
        ids[T // 2] = Eg + 1            # a token without a valid route
    counts, offsets, srt, slot = oracle.prepare_routes(ids, E, off, bm)
    gc, go, gs, gsl = binding.prepare_routes(torch.from_numpy(ids).cuda(), E, off, bm,
                                             chunked=chunked)
    torch.cuda.synchronize()
    total = int(offsets[-1])
    np.testing.assert_array_equal(gc.cpu().numpy(), counts)
    np.testing.assert_array_equal(go.cpu().numpy(), offsets)
    np.testing.assert_array_equal(gs.cpu().numpy()[:total], srt)
    np.testing.assert_array_equal(gsl.cpu().numpy(), slot)


def test_route_prep_skewed_and_local_share():
    for name, T in (("relu2_skew", 1024), ("deepseek_local", 512)):
        wl = synth.WORKLOADS[name]
        tok = synth.make_tokens(wl, T)
        ids = tok.topk_ids.numpy()
        counts, offsets, srt, slot = oracle.prepare_routes(ids, wl.num_experts, 0, 64)
        gc, go, gs, gsl = binding.prepare_routes(tok.topk_ids.cuda(), wl.num_experts, 0, 64)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gc.cpu().numpy(), counts)
        np.testing.assert_array_equal(go.cpu().numpy(), offsets)
        np.testing.assert_array_equal(gs.cpu().numpy()[:int(offsets[-1])], srt)
        np.testing.assert_array_equal(gsl.cpu().numpy(), slot)


# ---------------------------------------------------------------------------
# forward parity, every variant on the small gated workload
# ---------------------------------------------------------------------------

VARIANTS = ([dict(force_path=2), dict(force_path=1)]
            + [dict(force_path=1, force_splitk=sk) for sk in (1, 2)])


@pytest.mark.parametrize("force", VARIANTS, ids=lambda f: "-".join(f"{k}{v}" for k, v in f.items()))
def test_tiny_all_variants(force):
    wl = synth.WORKLOADS["tiny"]
    Wc, Wg = weights("tiny")
    tc = tokens(wl, 16)
    out = forward(wl, Wg, tc.to("cuda"), **force)
    assert_close(out, oracle_out(wl, Wc, tc), f"tiny {force}")


@pytest.mark.parametrize("name,T", [
    ("kimi_tp8", 1), ("kimi_tp8", 8), ("kimi_tp8", 16), ("kimi_tp8", 32), ("deepseek_local", 1),
    ("deepseek_local", 8), ("deepseek_local", 16), ("per_channel", 1), ("per_channel", 8),
    ("per_channel", 32), ("relu2_skew", 32)])
def test_configs_small_token_counts(name, T):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tc = tokens(wl, T)
    out = forward(wl, Wg, tc.to("cuda"))
    assert_close(out, oracle_out(wl, Wc, tc), f"{name} T={T}")


@pytest.mark.parametrize("name,T,force", [
    ("kimi_tp8", 8, dict(force_path=1)), ("kimi_tp8", 4, dict(force_path=2)),
    ("kimi_tp8", 8, dict(force_path=1, force_splitk=2)),
    ("kimi_tp8", 32, dict(force_path=1, force_splitk=1)),
    ("kimi_tp8", 32, dict(force_path=1, force_splitk=2)),
    ("kimi_tp8", 256, dict(force_path=1, force_splitk=1)),
    ("per_channel", 8, dict(force_path=1)),
    ("per_channel", 8, dict(force_path=1, force_splitk=1)),
    ("per_channel", 8, dict(force_path=1, force_splitk=2)),
    ("per_channel", 8, dict(force_path=2)),
    ("relu2_skew", 8, dict(force_path=2)),
    ("relu2_skew", 32, dict(force_path=1, force_splitk=1)),
    ("relu2_skew", 32, dict(force_path=1, force_splitk=2)),
    ("deepseek_local", 16, dict(force_path=1, force_splitk=1)),
    ("deepseek_local", 16, dict(force_path=1, force_splitk=2)),
    ("deepseek_local", 1, dict(force_path=2)),
    ("kimi_tp8", 16, dict(force_path=2)), ("kimi_tp8", 16, dict(force_path=1)),
    ("deepseek_local", 16, dict(force_path=1)), ("tiny", 64, dict(force_path=2)),
    # the automatic plan at the edges of the small-batch rule
    ("relu2_skew", 1, dict()), ("relu2_skew", 12, dict()), ("deepseek_local", 12, dict()),
    ("per_channel", 16, dict()), ("per_channel", 24, dict()), ("kimi_tp8", 48, dict()),
    ("kimi_tp8", 64, dict())])
def test_config_variants(name, T, force):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tc = tokens(wl, T)
    out = forward(wl, Wg, tc.to("cuda"), **force)
    assert_close(out, oracle_out(wl, Wc, tc), f"{name} T={T} {force}")


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _small(name="tiny"):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    return wl, Wc, Wg


def test_zero_tokens():
    wl, Wc, Wg = _small()
    tok = tokens(wl, 0, "cuda")
    out = forward(wl, Wg, tok)
    assert out.shape == (0, wl.hidden)


@pytest.mark.parametrize("path", [1, 2])
def test_invalid_routes_and_empty_tokens(path):
    wl, Wc, Wg = _small()
    tc = tokens(wl, 16)
    ids = tc.topk_ids.clone()
    ids[0, :] = -1                    # no valid route
    ids[3, 1] = wl.num_experts        # one past the end
    ids[5, 0] = 2 ** 31 - 1
    ids[7, :] = -(2 ** 31)
    tc = synth.Tokens(tc.x, ids, tc.topk_weights)
    out = forward(wl, Wg, tc.to("cuda"), force_path=path)
    ref = oracle_out(wl, Wc, tc)
    assert_close(out, ref, "invalid routes")
    o = out.cpu()
    assert (o[0] == 0).all() and (o[7] == 0).all()
    assert not torch.signbit(o[0].float()).any()


@pytest.mark.parametrize("path", [1, 2])
def test_all_routes_invalid_gives_zeros(path):
    wl, Wc, Wg = _small()
    tc = tokens(wl, 16)
    ids = torch.full_like(tc.topk_ids, 100)
    out = forward(wl, Wg, synth.Tokens(tc.x, ids, tc.topk_weights).to("cuda"), force_path=path)
    assert (out.cpu() == 0).all()


def test_single_expert_receives_everything():
    wl, Wc, Wg = _small()
    tc = tokens(wl, 32)
    ids = torch.full_like(tc.topk_ids, 3)       # duplicate ids: each route counts
    tc = synth.Tokens(tc.x, ids, tc.topk_weights)
    ref = oracle_out(wl, Wc, tc)
    for sk in (1, 2):
        out = forward(wl, Wg, tc.to("cuda"), force_path=1, force_splitk=sk)
        assert_close(out, ref, f"one expert force_splitk={sk}")
    out = forward(wl, Wg, tc.to("cuda"), force_path=2)           # 64 rows, 16 passes of 4
    assert_close(out, ref, "one expert small-batch path")
    # 128 routes, the expert's rows in both halves of the two ballots
    tc = tokens(wl, 64)
    ids = torch.full_like(tc.topk_ids, 3)
    ids[5, 0] = 1                                 # another expert between them
    tc = synth.Tokens(tc.x, ids, tc.topk_weights)
    out = forward(wl, Wg, tc.to("cuda"), force_path=2)
    assert_close(out, oracle_out(wl, Wc, tc), "one expert, 128 routes, small-batch path")


def test_small_batch_more_distinct_experts_than_expected():
    """When far fewer distinct local experts than routes are expected (here 8
    local of 512 global experts: one distinct local expert expected at 32
    tokens), the small-batch gate/up grid holds a few workgroup rows; when
    every route is local, each row takes several of the 8 experts in turn."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny_g512", num_global_experts=512)
    Wc = synth.make_weights(wl, device="cpu")
    Wg = Wc.to("cuda")
    for T in (16, 32):
        tc = tokens(wl, T)
        ids = (torch.arange(T * wl.top_k, dtype=torch.int32) % wl.num_experts).view(T, wl.top_k)
        tc = synth.Tokens(tc.x, ids, tc.topk_weights)
        assert binding.get_plan(binding.desc_for(wl, T)).path == 2
        out = forward(wl, Wg, tc.to("cuda"))
        assert_close(out, oracle_out(wl, Wc, tc), f"all routes local, T={T}")


def test_small_batch_expert_first_seen_past_route_64():
    """An expert whose first route lies past route 64 (owned through the second
    ballot), one spanning both halves, and invalid routes in both halves."""
    wl, Wc, Wg = _small()
    tc = tokens(wl, 64)                           # top-2: 128 routes
    ids = torch.full_like(tc.topk_ids, 2)
    ids.view(-1)[70:] = 5                         # expert 5 first seen at route 70
    ids.view(-1)[40:80:7] = 6                     # expert 6 in both halves
    ids.view(-1)[3] = -1
    ids.view(-1)[100] = 99                        # invalid routes
    tc = synth.Tokens(tc.x, ids, tc.topk_weights)
    out = forward(wl, Wg, tc.to("cuda"), force_path=2)
    assert_close(out, oracle_out(wl, Wc, tc), "experts past route 64")


def test_activations_beyond_fp16_range():
    """bf16 activations of magnitude 2^16 and more in tiles of several subtiles
    on the opted-in fp16 route (whose fp16 staging cannot hold them): those tiles are
    rerun with per-group scaling, so the affected rows stay exact and the
    others are untouched.  Without the rerun, 1e6 would be clamped to 65504."""
    wl = synth.WORKLOADS["tiny"]
    Wc, Wg = weights("tiny")
    tc = tokens(wl, 256)          # 512 routes over 8 experts: 64-row tiles of 4 subtiles
    x = tc.x.clone()
    big_rows = [3, 100, 200]
    x[3, 7] = 3.0e5
    x[100, 0] = -7.0e4
    x[200, 255] = 1.0e6
    t2 = synth.Tokens(x, tc.topk_ids, tc.topk_weights)
    ref = oracle_out(wl, Wc, t2)
    assert binding.get_plan(binding.desc_for(wl, 256, force_path=1, fp16_route=1)).fp16_route == 3
    out = forward(wl, Wg, t2.to("cuda"), force_path=1, fp16_route=1).cpu()
    rest = [r for r in range(256) if r not in big_rows]
    assert_close(out[rest], ref[rest], "tiny T=256, rows without large activations")
    for r in big_rows:
        nrmse, _ = errors(out[r], ref[r])
        assert nrmse <= 5e-3, (r, nrmse)


@pytest.mark.parametrize("inter", [384, 256], ids=["streaming-down", "resident-down"])
def test_fp16_route_rerun_flags(inter):
    """The down GEMM's fp16-route launch (the streaming tile kernel for
    I = 384, the resident one for I = 256) writes one flag per workgroup: all
    zero for ordinary activations, and set for the tiles whose staged
    activations reach 2^16 (large x rows make large silu(gate) * up), which
    the rerun launch then recomputes per group.  The workspace starts filled
    with 0xFF, so every flag having been written is checked too."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name=f"tiny_i{inter}", inter=inter)
    Wc = synth.make_weights(wl, device="cpu")
    Wg = Wc.to("cuda")
    tc = tokens(wl, 256)
    d = binding.desc_for(wl, 256, force_path=1, fp16_route=1)
    pl = binding.get_plan(d)
    assert pl.fp16_route == 3 and pl.rerun_flags_down > 0
    ws = torch.empty(binding.workspace_size(d), dtype=torch.uint8, device="cuda")
    off, n = pl.rerun_flags_offset + 4 * pl.rerun_flags_up, pl.rerun_flags_down

    def run(t):
        ws.fill_(0xFF)
        out = forward(wl, Wg, t.to("cuda"), force_path=1, fp16_route=1, workspace=ws).cpu()
        return out, ws[off:off + 4 * n].view(torch.int32).cpu()

    out, flags = run(tc)
    assert_close(out, oracle_out(wl, Wc, tc), "tiny T=256, flags run")
    assert int(flags.abs().sum()) == 0, flags
    x = tc.x.clone()
    x[3, 7] = 3.0e5
    x[200, 255] = 1.0e6
    t2 = synth.Tokens(x, tc.topk_ids, tc.topk_weights)
    out, flags = run(t2)
    assert bool(((flags == 0) | (flags == 1)).all()), flags
    assert int(flags.sum()) >= 1
    ref = oracle_out(wl, Wc, t2)
    for r in range(256):
        nrmse, _ = errors(out[r], ref[r])
        assert nrmse <= 5e-3, (r, nrmse)


@pytest.mark.parametrize("inter", [384, 256], ids=["streaming-down", "resident-down"])
@pytest.mark.parametrize("which,factor", [("w13", 2.0 ** -12), ("w2", 2.0 ** -12),
                                          ("w13", 2.0 ** 19), ("w2", 2.0 ** 19)],
                         ids=["w13-tiny", "w2-tiny", "w13-huge", "w2-huge"])
def test_fp16_route_scales_outside_exact_range(inter, which, factor):
    """The fp16 route forms q * s exactly only for 2^-17 <= |s| <= 2720 (or
    s = 0).  Scales multiplied by 2^-12 (all below 2^-17) or by 2^19 (1650
    to 7600, across the upper bound) must send the affected workgroups to the
    per-group rerun: every output row stays within the tolerance of the
    oracle, relative to its own size.  For w13 the tokens are divided by the
    same power of two, so that the activations between the two GEMMs keep
    their ordinary size (tiny activations are the route's other limit)."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name=f"tiny_i{inter}", inter=inter)
    Wc = synth.make_weights(wl, device="cpu")
    sc = getattr(Wc, f"{which}_scales")
    setattr(Wc, f"{which}_scales", (sc.float() * factor).to(sc.dtype))  # exact: a power of two
    tc = tokens(wl, 256)
    if which == "w13":
        tc = synth.Tokens((tc.x.float() / factor).to(tc.x.dtype), tc.topk_ids, tc.topk_weights)
    d = binding.desc_for(wl, 256, force_path=1, fp16_route=1)
    pl = binding.get_plan(d)
    assert pl.fp16_route == 3
    ws = torch.full((binding.workspace_size(d),), 0xFF, dtype=torch.uint8, device="cuda")
    out = forward(wl, Wc.to("cuda"), tc.to("cuda"), force_path=1, fp16_route=1,
                  workspace=ws).cpu()
    ref = oracle_out(wl, Wc, tc)
    for r in range(256):
        nrmse, _ = errors(out[r], ref[r])
        assert nrmse <= 5e-3, (r, nrmse)
    if which == "w2":
        off, n = pl.rerun_flags_offset + 4 * pl.rerun_flags_up, pl.rerun_flags_down
        flags = ws[off:off + 4 * n].view(torch.int32).cpu()
        assert int(flags.sum()) >= 1
    else:
        off, n = pl.rerun_flags_offset, pl.rerun_flags_up
        flags = ws[off:off + 4 * n].view(torch.int32).cpu()
        assert int(flags.sum()) >= 1


def test_zero_group_scales_stay_on_fp16_route():
    """All-zero weight groups (zero-padded or pruned weights) have scale 0,
    which the fp16 route forms exactly: no workgroup is sent to the rerun
    (every flag 0, each written: the workspace starts as 0xFF), and the
    output matches the oracle row by row."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny_i256", inter=256)
    Wc = synth.make_weights(wl, device="cpu")
    for name in ("w13", "w2"):
        sc = getattr(Wc, f"{name}_scales").clone()
        sc[:, :, ::3] = 0            # every third group of every row and expert
        setattr(Wc, f"{name}_scales", sc)
    tc = tokens(wl, 256)
    d = binding.desc_for(wl, 256, force_path=1, fp16_route=1)
    pl = binding.get_plan(d)
    assert pl.fp16_route == 3
    ws = torch.full((binding.workspace_size(d),), 0xFF, dtype=torch.uint8, device="cuda")
    out = forward(wl, Wc.to("cuda"), tc.to("cuda"), force_path=1, fp16_route=1,
                  workspace=ws).cpu()
    n = pl.rerun_flags_up + pl.rerun_flags_down
    off = pl.rerun_flags_offset
    flags = ws[off:off + 4 * n].view(torch.int32).cpu()
    assert int(flags.abs().sum()) == 0, flags
    assert_close(out, oracle_out(wl, Wc, tc), "zero groups on the fp16 route")


def test_rows_of_tiny_activations_default_plan_exact():
    """Rows whose activations all lie far below 2^-14 (x scaled by 2^-20): the
    default plan (fp16 route off) forms every product with per-group scaling,
    so every row, tiny or not, stays within the tolerance of the oracle
    relative to its own size, at a token count where the opted-in route
    would be taken."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny_i256", inter=256)
    Wc = synth.make_weights(wl, device="cpu")
    tc = tokens(wl, 256)
    x = tc.x.clone()
    tiny_rows = [5, 77, 200]
    x[tiny_rows] = (x[tiny_rows].float() * 2.0 ** -20).to(x.dtype)
    t2 = synth.Tokens(x, tc.topk_ids, tc.topk_weights)
    assert binding.get_plan(binding.desc_for(wl, 256, force_path=1, fp16_route=1)).fp16_route == 3
    assert binding.get_plan(binding.desc_for(wl, 256, force_path=1)).fp16_route == 0
    out = forward(wl, Wc.to("cuda"), t2.to("cuda"), force_path=1).cpu()
    ref = oracle_out(wl, Wc, t2)
    assert_close(out, ref, "tiny rows, default plan")


@pytest.mark.parametrize("T,force", [(16, f) for f in VARIANTS] + [
    (256, dict(force_path=1)), (256, dict(force_path=1, fp16_route=1))],
                         ids=lambda v: v if isinstance(v, int) else
                         "-".join(f"{k}{x}" for k, x in v.items()))
def test_local_share_at_nonzero_offset(T, force):
    """Experts 8..15 of 24 are local (an expert-parallel share that is not
    the first): ids below 8 or from 16 on are other ranks' routes and add
    nothing.  At 256 tokens an opted-in fp16 route is taken (about 21 valid
    routes per local expert)."""
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny_off8", num_global_experts=24,
                             expert_offset=8)
    Wc = synth.make_weights(wl, device="cpu")
    tc = tokens(wl, T)
    ids = tc.topk_ids
    assert bool(((ids < 8) | (ids >= 16)).any()) and bool(((ids >= 8) & (ids < 16)).any())
    if T == 256:
        want = 3 if force.get("fp16_route") else 0
        assert binding.get_plan(binding.desc_for(wl, T, **force)).fp16_route == want
    out = forward(wl, Wc.to("cuda"), tc.to("cuda"), **force)
    assert_close(out, oracle_out(wl, Wc, tc), f"offset 8 of 24, T={T} {force}")


POISON_CASES = [
    ("tiny", 16, dict(force_path=2)), ("tiny", 16, dict(force_path=1)),
    ("tiny", 16, dict(force_path=1, force_splitk=1)),
    ("tiny", 16, dict(force_path=1, force_splitk=2)),
    ("kimi_tp8", 32, dict()),                         # automatic plan: split-K
    ("deepseek_local", 16, dict()),                   # automatic plan: streaming tiles
    ("deepseek_local", 16, dict(force_path=1, force_splitk=1)),  # split-K over column
                                                      # chunks, activation launch
    ("tiny", 256, dict(force_path=1, fp16_route=1)),
    ("kimi_tp8", 256, dict(fused_finalize=1)),        # arrival counters start as 0xFF..
    ("deepseek_local", 16, dict(force_path=1, fused_finalize=1)),  # tokens without local routes
]


@pytest.mark.parametrize("name,T,force", POISON_CASES,
                         ids=lambda v: "-".join(f"{k}{x}" for k, x in v.items())
                         if isinstance(v, dict) else str(v))
def test_poisoned_workspace_and_output(name, T, force):
    """Workspace and output filled with NaN patterns before the call: nothing
    uninitialised may leak (empty split-K partitions, padding rows, FP32
    partials of routes that a chunk never touched)."""
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tc = tokens(wl, T)
    tg = tc.to("cuda")
    ref = oracle_out(wl, Wc, tc)
    d = binding.desc_for(wl, T, **force)
    if name == "kimi_tp8" and T == 32:
        assert binding.get_plan(d).splitk_chunks > 0
    ws = torch.full((binding.workspace_size(d),), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.full((T, wl.hidden), float("nan"), dtype=wl.dtype, device="cuda")
    binding.forward_workload(wl, Wg, tg, out=out, workspace=ws, **force)
    torch.cuda.synchronize()
    assert_close(out, ref, f"poisoned {name} T={T} {force}")


def test_workspace_reuse_across_token_counts():
    """One workspace and one output buffer reused over token counts that fill
    64-row tiles exactly, then leave ragged padded tails, then fill them again
    (aligned -> padded -> aligned): every call matches a call on a fresh
    NaN-poisoned workspace bit for bit, and the oracle."""
    wl = synth.WORKLOADS["tiny"]
    Wc, Wg = weights("tiny")
    seq = [256, 100, 256, 37, 128]           # 8 experts, top-2: 64, ~25, 64, ~9, 32 per expert
    big = max(binding.workspace_size(binding.desc_for(wl, t)) for t in seq)
    ws = torch.full((big,), 0xFF, dtype=torch.uint8, device="cuda")
    obuf = torch.full((max(seq) * wl.hidden,), float("nan"), dtype=wl.dtype, device="cuda")
    for T in seq:
        tc = tokens(wl, T)
        tg = tc.to("cuda")
        out = obuf[:T * wl.hidden].view(T, wl.hidden)
        binding.forward_workload(wl, Wg, tg, out=out, workspace=ws)
        fresh_ws = torch.full((binding.workspace_size(binding.desc_for(wl, T)),), 0xFF,
                              dtype=torch.uint8, device="cuda")
        fresh = binding.forward_workload(wl, Wg, tg, workspace=fresh_ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), fresh.view(torch.int16)), T
        assert_close(out, oracle_out(wl, Wc, tc), f"reuse T={T}")


def test_reduction_slices_cover_every_block():
    """The small-batch gate/up kernel splits the reduction over 8 waves in
    128-blocks; with H = 256 six waves get nothing and must add exact zeros."""
    wl, Wc, Wg = _small()
    tc = tokens(wl, 16)
    pl = binding.get_plan(binding.desc_for(wl, 16, force_path=2))
    assert pl.k_slice == 128
    out = forward(wl, Wg, tc.to("cuda"), force_path=2)
    assert_close(out, oracle_out(wl, Wc, tc), "H=256 over 8 waves")


@pytest.mark.parametrize("per_channel,gated,dtype", [
    (False, True, torch.bfloat16), (True, True, torch.bfloat16),
    (False, False, torch.float16), (True, False, torch.float16)])
def test_ragged_reduction_tails(per_channel, gated, dtype):
    """H = 320 and I = 192 end both reductions in a half (64-wide) block; with
    4 experts, T = 150 fills some experts past one 64-row tile (a full tile and
    a 1-subtile tail), T = 40 leaves 2 active subtiles per tile, T = 20 runs the
    small-batch path."""
    wl = synth.custom("tails", E=4, H=320, I=192, K=2, gated=gated, per_channel=per_channel,
                      dtype=dtype, seed=5)
    Wc = synth.make_weights(wl, device="cpu")
    Wg = Wc.to("cuda")
    for T, force in ((150, dict(force_path=1, force_splitk=2)),
                     (150, dict(force_path=1, force_splitk=1)), (40, dict(force_path=1)),
                     (40, dict(force_path=1, force_splitk=1)), (20, dict(force_path=2))):
        tc = tokens(wl, T)
        out = forward(wl, Wg, tc.to("cuda"), **force)
        assert_close(out, oracle_out(wl, Wc, tc), f"tails T={T} {force}")


@pytest.mark.parametrize("H,I,gated,dtype", [
    (6144, 192, True, torch.bfloat16), (320, 6144, False, torch.float16),
    (5760, 320, True, torch.bfloat16)], ids=["up-phases", "down-phases", "up-pair-scales"])
def test_long_reductions_scale_staging(H, I, gated, dtype):
    """For tiles of one active subtile the streaming tile kernel stages group
    scales in LDS: the whole reduction up to 176 groups, else in phases of
    112 groups when K / 32 is a multiple of 8 (6144: 112 + 80, the up
    projection prefetching, the down projection loading at the phase
    boundary), else fetched with the weights (5760: 180 groups), as they are
    for tiles of more subtiles.  T = 150 gives each expert a full tile and a
    one-subtile tail, T = 12 one-subtile tiles only, T = 40 two subtiles."""
    wl = synth.custom("scales", E=4, H=H, I=I, K=2, gated=gated, per_channel=False,
                      dtype=dtype, seed=11)
    Wc = synth.make_weights(wl, device="cpu")
    Wg = Wc.to("cuda")
    for T in (150, 12, 40):
        tc = tokens(wl, T)
        out = forward(wl, Wg, tc.to("cuda"), force_path=1, force_splitk=2)
        assert_close(out, oracle_out(wl, Wc, tc), f"H={H} I={I} T={T}")


# ---------------------------------------------------------------------------
# determinism, invariances, graph replay
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,T", [("tiny", 16), ("kimi_tp8", 8), ("kimi_tp8", 32)])
def test_bitwise_repeatable(name, T):
    wl = synth.WORKLOADS[name]
    _, Wg = weights(name)
    tg = tokens(wl, T, "cuda")
    a = forward(wl, Wg, tg)
    for _ in range(3):
        b = forward(wl, Wg, tg)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("path", [1, 2])
def test_gpu_invariances_bitwise(path):
    wl, Wc, Wg = _small()
    tc = tokens(wl, 16)
    base = forward(wl, Wg, tc.to("cuda"), force_path=path).cpu()
    # routing weights x2 -> output x2 exactly
    t2 = synth.Tokens(tc.x, tc.topk_ids, tc.topk_weights * 2)
    o2 = forward(wl, Wg, t2.to("cuda"), force_path=path).cpu()
    assert torch.equal(o2.float(), base.float() * 2)
    # token permutation -> output permutation exactly
    perm = torch.randperm(16, generator=torch.Generator().manual_seed(1))
    tp = synth.Tokens(tc.x[perm].contiguous(), tc.topk_ids[perm].contiguous(),
                      tc.topk_weights[perm].contiguous())
    op = forward(wl, Wg, tp.to("cuda"), force_path=path).cpu()
    assert torch.equal(op.view(torch.int16), base[perm].view(torch.int16))


GRAPH_CASES = [("kimi_tp8", 1, dict()), ("kimi_tp8", 32, dict()),
               ("kimi_tp8", 256, dict(fp16_route=1)), ("kimi_tp8", 1024, dict(fp16_route=1)),
               ("per_channel", 8, dict()), ("per_channel", 256, dict()),
               ("relu2_skew", 32, dict()), ("relu2_skew", 1024, dict()),
               ("deepseek_local", 16, dict()), ("kimi_tp8", 256, dict(fused_finalize=1)),
               ("relu2_skew", 1024, dict(fused_finalize=1))]


@pytest.mark.parametrize("name,T,force", GRAPH_CASES,
                         ids=lambda v: "-".join(f"{k}{x}" for k, x in v.items())
                         if isinstance(v, dict) else str(v))
def test_hip_graph_replay(name, T, force):
    """The forward captured in a HIP graph replays to the eager result bit for
    bit, three times, with eager work and synchronizations between replays
    (small batch, split-K, streaming tiles, per-channel, ReLU^2 fp16, the
    opted-in fp16 route with its rerun launches)."""
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tg = tokens(wl, T, "cuda")
    d = binding.desc_for(wl, T, **force)
    pl = binding.get_plan(d)
    sys_msg = f"{name} T={T} plan path={pl.path} splitk={pl.splitk_chunks} fp16={pl.fp16_route}"
    print(sys_msg, flush=True)
    ws = torch.empty(binding.workspace_size(d), dtype=torch.uint8, device="cuda")
    out = torch.empty(T, wl.hidden, dtype=wl.dtype, device="cuda")
    eager = forward(wl, Wg, tg, **force).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.forward_workload(wl, Wg, tg, out=out, workspace=ws, **force)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.forward_workload(wl, Wg, tg, out=out, workspace=ws, **force)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
        forward(wl, Wg, tg, **force)              # eager work between replays
    if T <= 32:
        assert_close(out, oracle_out(wl, Wc, tokens(wl, T)), f"graph {name} T={T}")


@pytest.mark.parametrize("name,T", [("tiny", 256), ("kimi_tp8", 32), ("kimi_tp8", 256),
                                    ("kimi_tp8", 2048), ("deepseek_local", 16),
                                    ("deepseek_local", 512), ("per_channel", 256),
                                    ("relu2_skew", 1024)])
def test_fused_finalize_matches_separate_launch(name, T):
    """The fused finalize (the combine inside the down launch: the workgroup
    that completes a token's routes for a column chunk sums them in ascending
    k) gives the same bits as the default combine launch of its own, for the
    resident (I <= 256) and the streaming down kernels, tokens without local
    routes included, and repeats bitwise (the arrival order varies from run
    to run)."""
    wl = synth.WORKLOADS[name]
    _, Wg = weights(name)
    tg = tokens(wl, T, "cuda")
    grouped = dict(force_path=1)  # the mode belongs to the grouped path
    assert binding.get_plan(binding.desc_for(wl, T, **grouped)).fused_combine == 0
    assert binding.get_plan(binding.desc_for(wl, T, fused_finalize=1, **grouped)).fused_combine == 1
    sep = forward(wl, Wg, tg, **grouped)
    for _ in range(3):
        d = binding.desc_for(wl, T, fused_finalize=1, **grouped)
        ws = torch.full((binding.workspace_size(d),), 0xFF, dtype=torch.uint8, device="cuda")
        out = torch.full((T, wl.hidden), float("nan"), dtype=wl.dtype, device="cuda")
        binding.forward_workload(wl, Wg, tg, out=out, workspace=ws, fused_finalize=1, **grouped)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), sep.view(torch.int16)), name
