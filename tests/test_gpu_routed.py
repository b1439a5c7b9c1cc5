"""GPU parity of the forward with the router fused in (w4a16_moe_forward_routed)
and of routing fused with route preparation (w4a16_moe_route_and_prepare),
through the C ABI, against the CPU oracle (oracle_route_topk, then
oracle_prepare_routes and the oracle forward on the oracle's routes): ids and
route tables bit-exact, weights within a relative 1e-5, outputs within the
NRMSE bar; and against the unfused device path (standalone router, then the
forward): identical bits."""
import numpy as np
import pytest
import torch

import oracle
from moe_check import assert_close, oracle_out, tokens, weights
from w4a16_mixture_experts_amd import binding, synth

pytestmark = pytest.mark.gpu


def _oracle_routes(logits: np.ndarray, K: int, renorm=False):
    return oracle.route_topk(logits, K, renormalize=renorm)


# (workload, T): small-batch path (routing inside the gate/up kernel up to 16
# routes, else the router kernel first), one preparation workgroup routing
# up to 16 tokens itself, and the router kernel before the preparation
# beyond that (one workgroup or chunked)
CASES = [("kimi_tp8", 1), ("kimi_tp8", 2), ("kimi_tp8", 8), ("kimi_tp8", 32), ("kimi_tp8", 256),
         ("kimi_tp8", 2048), ("deepseek_local", 1), ("deepseek_local", 16),
         ("deepseek_local", 512), ("per_channel", 8), ("per_channel", 256),
         ("relu2_skew", 32), ("relu2_skew", 1024), ("relu2_skew", 4096), ("tiny", 16)]


@pytest.mark.parametrize("name,T", CASES)
def test_routed_forward(name, T):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tc = tokens(wl, T)
    tg = tc.to("cuda")
    logits = tc.logits.numpy()
    out, ids, wts = binding.forward_workload_routed(wl, Wg, tg)
    torch.cuda.synchronize()
    ref_i, ref_w = _oracle_routes(logits, wl.top_k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_i)
    np.testing.assert_allclose(wts.cpu().numpy(), ref_w, rtol=1e-5, atol=1e-8)
    # the unfused device path: the standalone router, then the forward
    ids2, wts2 = binding.route_topk(tg.logits, wl.top_k)
    assert torch.equal(ids, ids2) and torch.equal(wts.view(torch.int32), wts2.view(torch.int32))
    out2 = binding.forward_workload(wl, Wg, synth.Tokens(tg.x, ids2, wts2))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), (name, T)
    # the oracle forward on the oracle's routing
    t_or = synth.Tokens(tc.x, torch.from_numpy(ref_i), torch.from_numpy(ref_w))
    if T <= 256 or name == "deepseek_local":
        assert_close(out, oracle_out(wl, Wc, t_or), f"routed {name} T={T}")
    else:
        rows = sorted(set([0, T - 1] + np.random.default_rng(T).choice(T, 14, replace=False).tolist()))
        ref = oracle_out(wl, Wc, t_or, rows=rows)
        assert_close(out[torch.as_tensor(rows, device="cuda")], ref, f"routed {name} T={T} rows")


@pytest.mark.parametrize("name,T", [(n, T) for n, T in CASES if T > 1] + [
    ("kimi_tp8", 128), ("kimi_tp8", 12), ("relu2_skew", 16), ("kimi_tp8", 17)])
@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "one-chunk"])
def test_route_and_prepare_tables_bit_exact(name, T, chunked):
    wl = synth.WORKLOADS[name]
    tc = tokens(wl, T)
    logits = tc.logits.numpy()
    ids, wts, counts, offsets, srt, slot = binding.route_and_prepare(
        tc.logits.cuda(), wl.top_k, wl.num_experts, wl.expert_offset, 64, chunked=chunked)
    torch.cuda.synchronize()
    ref_i, ref_w = _oracle_routes(logits, wl.top_k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_i)
    np.testing.assert_allclose(wts.cpu().numpy(), ref_w, rtol=1e-5, atol=1e-8)
    c, o, s, sl = oracle.prepare_routes(ref_i, wl.num_experts, wl.expert_offset, 64)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    np.testing.assert_array_equal(srt.cpu().numpy()[:int(o[-1])], s)
    np.testing.assert_array_equal(slot.cpu().numpy(), sl)


@pytest.mark.parametrize("T,Eg,K,E,off", [(100, 384, 8, 384, 0), (7, 24, 3, 8, 8),
                                          (300, 60, 4, 60, 0), (1000, 1024, 1, 1024, 0),
                                          (40, 128, 6, 32, 96)])
@pytest.mark.parametrize("renorm", [False, True])
def test_route_and_prepare_shapes_and_renorm(T, Eg, K, E, off, renorm):
    """Local shares at an offset, K = 1 and K = 3, 1024 global experts, and
    renormalized weights, with masked (-inf) experts and an all -inf token."""
    rng = np.random.default_rng(T + Eg + K)
    logits = rng.standard_normal((T, Eg)).astype(np.float32)
    logits[:, Eg - 1] = -np.inf
    logits[T // 2] = -np.inf
    ids, wts, counts, offsets, srt, slot = binding.route_and_prepare(
        torch.from_numpy(logits).cuda(), K, E, off, 64, renormalize=renorm)
    torch.cuda.synchronize()
    ref_i, ref_w = _oracle_routes(logits, K, renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_i)
    np.testing.assert_allclose(wts.cpu().numpy(), ref_w, rtol=1e-5, atol=1e-8)
    c, o, s, sl = oracle.prepare_routes(ref_i, E, off, 64)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    np.testing.assert_array_equal(srt.cpu().numpy()[:int(o[-1])], s)
    np.testing.assert_array_equal(slot.cpu().numpy(), sl)


def test_routed_forward_renormalized_and_zero_tokens():
    wl = synth.WORKLOADS["deepseek_local"]
    Wc, Wg = weights("deepseek_local")
    tc = tokens(wl, 16)
    out, ids, wts = binding.forward_workload_routed(wl, Wg, tc.to("cuda"), renormalize=True)
    torch.cuda.synchronize()
    ref_i, ref_w = _oracle_routes(tc.logits.numpy(), wl.top_k, True)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_i)
    np.testing.assert_allclose(wts.cpu().numpy(), ref_w, rtol=1e-5, atol=1e-8)
    t_or = synth.Tokens(tc.x, torch.from_numpy(ref_i), torch.from_numpy(ref_w))
    assert_close(out, oracle_out(wl, Wc, t_or), "routed renormalized")
    t0 = tokens(wl, 0, "cuda")
    out0, ids0, _ = binding.forward_workload_routed(wl, Wg, t0)
    assert out0.shape == (0, wl.hidden) and ids0.shape == (0, wl.top_k)


@pytest.mark.parametrize("name,T", [("kimi_tp8", 1), ("kimi_tp8", 256), ("relu2_skew", 1024)])
def test_routed_forward_graph_replay(name, T):
    wl = synth.WORKLOADS[name]
    _, Wg = weights(name)
    tg = tokens(wl, T, "cuda")
    out = torch.empty(T, wl.hidden, dtype=wl.dtype, device="cuda")
    ids = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    wts = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    d = binding.desc_for(wl, T)
    ws = torch.empty(binding.workspace_size(d), dtype=torch.uint8, device="cuda")
    eager, ei, ew = binding.forward_workload_routed(wl, Wg, tg)
    eager, ei, ew = eager.clone(), ei.clone(), ew.clone()

    def run():
        binding.forward_workload_routed(wl, Wg, tg, out=out, ids_out=(ids, wts), workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(3):
        out.zero_()
        ids.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
        assert torch.equal(ids, ei) and torch.equal(wts.view(torch.int32), ew.view(torch.int32))
        binding.forward_workload_routed(wl, Wg, tg)   # eager work between replays


@pytest.mark.parametrize("T,force", [(4, dict(force_path=2)), (200, dict(force_path=1)),
                                     (1500, dict(force_path=1))])
def test_routed_forward_many_global_experts(T, force):
    """1000 global experts (more than the small-batch launch routes itself:
    the router kernel runs first there), 8 of them local at offset 0."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny_g1000", num_global_experts=1000)
    Wc = synth.make_weights(wl, device="cpu")
    Wg = Wc.to("cuda")
    tc = tokens(wl, T)
    out, ids, wts = binding.forward_workload_routed(wl, Wg, tc.to("cuda"), **force)
    torch.cuda.synchronize()
    ref_i, ref_w = _oracle_routes(tc.logits.numpy(), wl.top_k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_i)
    np.testing.assert_allclose(wts.cpu().numpy(), ref_w, rtol=1e-5, atol=1e-8)
    t_or = synth.Tokens(tc.x, torch.from_numpy(ref_i), torch.from_numpy(ref_w))
    assert_close(out, oracle_out(wl, Wc, t_or), f"routed 1000 global T={T}")
