"""Properties of the seeded input generator (shapes, routing recipe, skew)."""
import torch

from w4a16_mixture_experts_amd import synth


def test_routes_recipe_and_determinism():
    wl = synth.WORKLOADS["tiny"]
    a = synth.make_tokens(wl, 16)
    b = synth.make_tokens(wl, 16)
    assert torch.equal(a.topk_ids, b.topk_ids) and torch.equal(a.x, b.x)
    assert a.topk_ids.dtype == torch.int32 and a.topk_weights.dtype == torch.float32
    assert a.x.dtype == torch.bfloat16 and a.x.shape == (16, 256)
    # top-k of a softmax: descending, distinct ids, no renormalisation (sum < 1)
    assert (a.topk_weights[:, :-1] >= a.topk_weights[:, 1:]).all()
    assert all(len(set(r.tolist())) == wl.top_k for r in a.topk_ids)
    assert (a.topk_weights.sum(1) < 1).all()


def test_local_share_routes_over_global_experts():
    wl = synth.WORKLOADS["deepseek_local"]
    tok = synth.make_tokens(wl, 64)
    assert int(tok.topk_ids.max()) < 256 and int(tok.topk_ids.min()) >= 0
    local = (tok.topk_ids < 32).float().mean().item()
    assert 0.05 < local < 0.25            # about 32/256 of the routes are local


def test_relu2_skew():
    wl = synth.WORKLOADS["relu2_skew"]
    tok = synth.make_tokens(wl, 1024)
    ids = tok.topk_ids
    assert not ((ids % 16) == 15).any()                       # masked experts get nothing
    hot = (ids < 4).float().mean().item()
    assert abs(hot - 0.25) < 0.01 and abs(tok.hot_share - hot) < 1e-9
    assert tok.x.dtype == torch.float16


def test_weight_shapes():
    for name, wl in synth.WORKLOADS.items():
        if wl.num_experts * wl.hidden * wl.n1 > 2e7:
            continue
        W = synth.make_weights(wl)
        E, H, I, N1 = wl.num_experts, wl.hidden, wl.inter, wl.n1
        if wl.per_channel:
            assert W.w13_packed.shape == (E, N1 // 2, H) and W.w13_scales.shape == (E, N1)
            assert W.w2_packed.shape == (E, H // 2, I) and W.w2_scales.shape == (E, H)
        else:
            assert W.w13_packed.shape == (E, N1, H // 2)
            assert W.w13_scales.shape == (E, N1, H // 32)
            assert W.w2_packed.shape == (E, H, I // 2) and W.w2_scales.shape == (E, H, I // 32)
        assert W.w13_scales.dtype == wl.dtype
