"""GPU parity of the router (softmax over all global experts, top-k) through
the C ABI against the CPU oracle: expert ids bit-exact, weights within a
relative 1e-5 (FP32 exponentials and sums against the oracle's float64)."""
import numpy as np
import pytest
import torch

import oracle
from moe_check import assert_close, forward, oracle_out, weights
from w4a16_mixture_experts_amd import binding, synth

pytestmark = pytest.mark.gpu


def _check(logits: np.ndarray, K: int, renorm: bool = False):
    ids, w = binding.route_topk(torch.from_numpy(logits).cuda(), K, renormalize=renorm)
    torch.cuda.synchronize()
    ref_i, ref_w = oracle.route_topk(logits, K, renormalize=renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_i)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=1e-5, atol=1e-8)
    return ids, w


@pytest.mark.parametrize("T,Eg,K", [(1, 384, 8), (8, 384, 8), (2048, 384, 8), (33, 256, 8),
                                    (16, 8, 2), (5, 60, 4), (7, 1024, 32), (3, 64, 64 // 2),
                                    (9, 65, 1), (4, 1, 1)])
@pytest.mark.parametrize("renorm", [False, True])
def test_route_topk_parity(T, Eg, K, renorm):
    rng = np.random.default_rng(T * 1000 + Eg + K)
    _check(rng.standard_normal((T, Eg)).astype(np.float32), K, renorm)


def test_route_topk_ties_and_masked_experts():
    # equal logits: ids ascending, weights 1/E
    _check(np.zeros((4, 384), np.float32), 8)
    # duplicated values across lanes and slots (ids e and e + 64 share a lane)
    rng = np.random.default_rng(7)
    logits = rng.integers(-3, 4, size=(64, 256)).astype(np.float32)
    _check(logits, 8)
    _check(logits, 8, renorm=True)
    # masked experts (-inf) as in the skewed ReLU^2 workload, and a token
    # whose logits are all -inf (zero weights, lowest ids)
    logits = rng.standard_normal((32, 128)).astype(np.float32)
    logits[:, 15::16] = -np.inf
    logits[5] = -np.inf
    _check(logits, 6)


def test_route_topk_zero_tokens_and_errors():
    ids, w = binding.route_topk(torch.zeros(0, 384, device="cuda"), 8)
    assert ids.shape == (0, 8) and w.shape == (0, 8)
    with pytest.raises(binding.W4A16Error):
        binding.route_topk(torch.zeros(2, 4, device="cuda"), 5)          # top_k > E_global
    with pytest.raises(binding.W4A16Error):
        binding.route_topk(torch.zeros(2, 1025, device="cuda"), 8)       # too many experts


def test_route_topk_bitwise_repeatable():
    logits = torch.from_numpy(np.random.default_rng(1).standard_normal((300, 384)).astype(
        np.float32)).cuda()
    a = binding.route_topk(logits, 8)
    for _ in range(3):
        b = binding.route_topk(logits, 8)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_route_then_forward():
    """Router on the GPU feeding the forward: same ids as the oracle's router,
    and the forward's output within the bar of the oracle's forward on the
    oracle's routing (the DeepSeek-like share: 256 global experts, 32 local)."""
    wl = synth.WORKLOADS["deepseek_local"]
    Wc, Wg = weights("deepseek_local")
    rng = np.random.default_rng(11)
    T = 64
    x = torch.from_numpy(rng.standard_normal((T, wl.hidden)).astype(np.float32)).to(wl.dtype)
    logits = rng.standard_normal((T, wl.num_global_experts)).astype(np.float32)
    ids, w = _check(logits, wl.top_k)
    ref_i, ref_w = oracle.route_topk(logits, wl.top_k)
    tg = synth.Tokens(x.cuda(), ids, w)
    out = forward(wl, Wg, tg)
    ref = oracle_out(wl, Wc, synth.Tokens(x, torch.from_numpy(ref_i), torch.from_numpy(ref_w)))
    assert_close(out, ref, "deepseek_local T=64 routed on the GPU")
