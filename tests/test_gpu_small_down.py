"""The small-batch down kernel's work items: only valid routes take (route,
256-wide slice) items, and a wave with more items than one loads its next
item while it computes the current one.  Tokens whose valid routes are
scattered over the top-k slots, item counts that are and are not multiples
of the 8 waves, and a token with no valid route, against the oracle."""
import pytest
import torch

from moe_check import assert_close, forward, oracle_out, tokens, weights
from w4a16_mixture_experts_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("I,per_channel,valid", [
    (2048, False, (0, 2, 5, 7)),     # 8 slices per route: 32 items, 4 per wave
    (1408, True, (1, 3, 6)),         # 6 slices: 18 items, 2 or 3 per wave
    (1408, False, (4,)),             # 6 items: two waves without an item
    (256, False, (7,)),              # one slice per route
    (256, False, tuple(range(8))),   # every route valid
])
def test_valid_route_items(I, per_channel, valid):
    wl = synth.custom("down_items", E=12, H=256, I=I, K=8, per_channel=per_channel, seed=5)
    Wc = synth.make_weights(wl, device="cpu")
    Wg = Wc.to("cuda")
    tc = tokens(wl, 4)
    ids = tc.topk_ids.clone()
    keep = torch.zeros(8, dtype=torch.bool)
    keep[list(valid)] = True
    bad = torch.tensor([-1, 99, 12, -5, 1000, -1, 13, 40], dtype=ids.dtype)
    ids[:3, ~keep] = bad[~keep]
    ids[3, :] = -1                                  # a token with no valid route
    tc = synth.Tokens(tc.x, ids, tc.topk_weights)
    out = forward(wl, Wg, tc.to("cuda"), force_path=2)
    assert not out[3].any()
    assert_close(out, oracle_out(wl, Wc, tc), f"I={I} valid={valid}")


@pytest.mark.parametrize("name,T", [("kimi_tp8", 7), ("kimi_tp8", 13), ("deepseek_local", 5),
                                    ("per_channel", 11), ("tiny", 9)])
def test_odd_token_counts_with_an_empty_token(name, T):
    """Odd token counts, one token's routes all invalid (its output row is
    zero and its down workgroups take no item)."""
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tc = tokens(wl, T)
    ids = tc.topk_ids.clone()
    ids[T // 2, :] = -1
    tc = synth.Tokens(tc.x, ids, tc.topk_weights)
    out = forward(wl, Wg, tc.to("cuda"), force_path=2)
    assert not out[T // 2].any()
    assert_close(out, oracle_out(wl, Wc, tc), f"{name} T={T} empty token")
