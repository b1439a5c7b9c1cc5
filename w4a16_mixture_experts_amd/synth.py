"""Seeded synthetic inputs for the local W4A16 MoE forward.

This module produces inputs only: packed INT4 expert weights with their 16-bit
scales, 16-bit activations and top-k routes.  It contains none of the forward
pass's arithmetic (no dequantization, GEMM, activation or combine); both the
HIP path and the CPU oracle consume exactly the bytes it returns.

Workloads (the pages' shapes, with synthetic data standing in for model
weights and router outputs):
  tiny            8 experts, H 256, I 384, top-2, bf16, group-32 along K
  kimi_tp8        384 experts, H 7168, I 256, top-8 (one TP8 shard of a
                  Kimi-like MoE; lmdeploy PR #4947, Benchmark)
  deepseek_local  32 local of 256 global experts, H 7168, I 2048, top-8
                  (single-GPU simulated EP8 share; flashinfer PR #5186,
                  Final performance)
  per_channel     60 experts, H 2048, I 1408, top-4, one scale per output
                  channel, INT4 packed along the output dim (TensorRT-LLM PR
                  #18313, Validation and Checkpoint format)
  relu2_skew      128 experts, H 2688, I 1856, top-6, non-gated ReLU^2, fp16,
                  skewed routing (TensorRT-LLM PR #18313, Validation)
  *_fp4           the Kimi shard and the DeepSeek share with FP4 weights:
                  MXFP4 (E2M1 codes, one power-of-two scale per 32 along K)
                  standing in for the NVFP4 weights flashinfer PR #5186 (Final
                  performance) measures, with 16-bit activations

Recipe (fixed here, stated in the design notes):
  weights   fp32 ~ N(0, 0.02), drawn per expert in ascending order (w13_e then
            w2_e) from a generator seeded with the workload seed; symmetric
            INT4, scale = absmax / 7 rounded to the 16-bit dtype,
            q = clamp(round_half_even(w / scale), -8, 7), q = 0 where the
            scale is 0; two values per byte, even index in the low nibble.
  tokens    a generator seeded with seed + T draws x ~ N(0, 1) (fp32, then
            rounded to the 16-bit dtype) and then router logits ~ N(0, 1)
            [T, E_global]; routing weights are softmax over all global experts,
            top-k (descending), no renormalisation; ids are int32.
  fp4       the same fp32 weights quantized to MXFP4 in blocks of 32 along K:
            exponent x = floor(log2(max |w|)) - 2, clamped to [-127, 127]
            (E8M0 code x + 127; an all-zero block gets code 0 and zero
            values), codes = w / 2^x rounded to the nearest E2M1 value (ties to
            the even mantissa bit, saturating at 6); the 16-bit scale is
            2^x, exact in bf16.
  skew      relu2_skew masks experts e % 16 == 15 (logit -inf, they receive no
            tokens) and adds a bias b to experts 0..3, with b found by
            bisection so that the share of routes on those four experts is the
            closest to 0.25.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

GROUP = 32


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_experts: int          # local experts E
    num_global_experts: int   # experts the router chooses from
    expert_offset: int        # first global id owned locally
    hidden: int               # H
    inter: int                # I
    top_k: int                # K
    gated: bool               # SiLU(gate)*up if True, ReLU^2 if False
    per_channel: bool         # one scale per output channel, packed along N
    dtype: torch.dtype        # activations, scales and output
    tokens: tuple             # token counts of the sweep
    seed: int
    skew: bool = False
    fp4: bool = False         # MXFP4 (E2M1) weights instead of INT4 (group layout)

    @property
    def n1(self) -> int:
        return 2 * self.inter if self.gated else self.inter


WORKLOADS = {
    "tiny": Workload("tiny", 8, 8, 0, 256, 384, 2, True, False, torch.bfloat16, (16,), 0),
    "kimi_tp8": Workload("kimi_tp8", 384, 384, 0, 7168, 256, 8, True, False, torch.bfloat16,
                         (1, 8, 32, 256, 1024, 2048), 20260908),
    "deepseek_local": Workload("deepseek_local", 32, 256, 0, 7168, 2048, 8, True, False,
                               torch.bfloat16, (1, 16, 128, 512, 2048), 20260908),
    "per_channel": Workload("per_channel", 60, 60, 0, 2048, 1408, 4, True, True, torch.bfloat16,
                            (1, 8, 256), 20260908),
    "relu2_skew": Workload("relu2_skew", 128, 128, 0, 2688, 1856, 6, False, False, torch.float16,
                           (32, 1024, 4096), 20260908, skew=True),
    "kimi_tp8_fp4": Workload("kimi_tp8_fp4", 384, 384, 0, 7168, 256, 8, True, False,
                             torch.bfloat16, (1, 8, 32, 256, 1024, 2048), 20260908, fp4=True),
    "deepseek_local_fp4": Workload("deepseek_local_fp4", 32, 256, 0, 7168, 2048, 8, True, False,
                                   torch.bfloat16, (1, 16, 128, 512, 2048), 20260908, fp4=True),
}


def custom(name="custom", *, E, H, I, K, gated=True, per_channel=False, dtype=torch.bfloat16,
           E_global=None, offset=0, seed=0, skew=False, fp4=False) -> Workload:
    """A workload of any shape (tests use small ones)."""
    return Workload(name, E, E_global or E, offset, H, I, K, gated, per_channel, dtype, (), seed,
                    skew, fp4)


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------

def _pack_pairs(lo: torch.Tensor, hi: torch.Tensor) -> torch.Tensor:
    """Two int8 tensors in [-8, 7] -> bytes (lo in the low nibble)."""
    return ((lo.to(torch.int16) & 0xF) | ((hi.to(torch.int16) & 0xF) << 4)).to(torch.uint8)


def _quant(w: torch.Tensor, amax: torch.Tensor, dtype: torch.dtype):
    s16 = (amax / 7.0).to(dtype)
    s = s16.float()
    safe = torch.where(s == 0, torch.ones_like(s), s)
    q = torch.clamp(torch.round(w / safe), -8, 7)
    q = torch.where(s == 0, torch.zeros_like(q), q).to(torch.int8)
    return q, s16


def quantize_matrix(w: torch.Tensor, per_channel: bool, dtype: torch.dtype):
    """fp32 [n_out, k_in] -> (packed uint8, scales 16-bit).

    group mode: packed [n_out, k_in/2] along K, scales [n_out, k_in/32]
    per-channel: packed [n_out/2, k_in] along N, scales [n_out]
    """
    n_out, k_in = w.shape
    if per_channel:
        amax = w.abs().amax(dim=1, keepdim=True)
        q, s16 = _quant(w, amax, dtype)
        packed = _pack_pairs(q[0::2, :], q[1::2, :])
        return packed.contiguous(), s16.reshape(n_out).contiguous()
    wg = w.reshape(n_out, k_in // GROUP, GROUP)
    amax = wg.abs().amax(dim=2, keepdim=True)
    q, s16 = _quant(wg, amax, dtype)
    q = q.reshape(n_out, k_in)
    packed = _pack_pairs(q[:, 0::2], q[:, 1::2])
    return packed.contiguous(), s16.reshape(n_out, k_in // GROUP).contiguous()


# magnitudes of the E2M1 codes 0..7 (bit 0 mantissa, bits 2..1 exponent with
# bias 1; exponent 0 subnormal)
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantize_mxfp4(w: torch.Tensor):
    """fp32 [n_out, k_in] -> (packed uint8 [n_out, k_in/2], E8M0 uint8 [n_out, k_in/32])."""
    n_out, k_in = w.shape
    wg = w.reshape(n_out, k_in // GROUP, GROUP)
    amax = wg.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                     # amax = m * 2^ex, m in [0.5, 1)
    zero = amax == 0
    x = torch.clamp(ex.to(torch.int32) - 3, -127, 127)   # floor(log2 amax) - 2
    x = torch.where(zero, torch.full_like(x, -127), x)
    scale = torch.ldexp(torch.ones_like(amax), x.to(torch.float32))
    v = wg / scale[..., None]
    grid = torch.tensor(E2M1_GRID, dtype=torch.float32, device=w.device)
    d = (v.abs()[..., None] - grid).abs()
    is_min = d == d.amin(dim=-1, keepdim=True)
    even = torch.tensor([True, False] * 4, device=w.device)
    cand = is_min & even
    idx = torch.where(cand.any(dim=-1), cand.to(torch.int8).argmax(dim=-1),
                      is_min.to(torch.int8).argmax(dim=-1))
    sign = (v < 0) | ((v == 0) & torch.signbit(v))
    code = (idx + 8 * sign.to(idx.dtype)).to(torch.int16)
    code = torch.where(zero[..., None], torch.zeros_like(code), code).reshape(n_out, k_in)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).to(torch.uint8)
    return packed.contiguous(), (x + 127).to(torch.uint8).contiguous()


def e8m0_to_h16(e8: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    """E8M0 codes -> the 16-bit scale 2^(e - 127) (must be exact in dtype)."""
    v = torch.ldexp(torch.ones(e8.shape, device=e8.device), e8.to(torch.float32) - 127)
    s = v.to(dtype)
    if not torch.equal(s.float(), v):
        raise ValueError(f"E8M0 scale not exact in {dtype}")
    return s


@dataclasses.dataclass
class Weights:
    w13_packed: torch.Tensor
    w13_scales: torch.Tensor
    w2_packed: torch.Tensor
    w2_scales: torch.Tensor

    def to(self, device) -> "Weights":
        return Weights(*(t.to(device) for t in dataclasses.astuple(self)))


def make_weights(wl: Workload, device="cpu", seed: Optional[int] = None,
                 std: float = 0.02) -> Weights:
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed if seed is None else seed)
    E, H, I, N1 = wl.num_experts, wl.hidden, wl.inter, wl.n1
    if wl.per_channel:
        w13p = torch.empty(E, N1 // 2, H, dtype=torch.uint8, device=device)
        w13s = torch.empty(E, N1, dtype=wl.dtype, device=device)
        w2p = torch.empty(E, H // 2, I, dtype=torch.uint8, device=device)
        w2s = torch.empty(E, H, dtype=wl.dtype, device=device)
    else:
        w13p = torch.empty(E, N1, H // 2, dtype=torch.uint8, device=device)
        w13s = torch.empty(E, N1, H // GROUP, dtype=wl.dtype, device=device)
        w2p = torch.empty(E, H, I // 2, dtype=torch.uint8, device=device)
        w2s = torch.empty(E, H, I // GROUP, dtype=wl.dtype, device=device)
    for e in range(E):
        w13 = torch.randn(N1, H, generator=g, device=device, dtype=torch.float32) * std
        w2 = torch.randn(H, I, generator=g, device=device, dtype=torch.float32) * std
        if wl.fp4:
            p13, e13 = quantize_mxfp4(w13)
            p2, e2 = quantize_mxfp4(w2)
            w13p[e], w13s[e] = p13, e8m0_to_h16(e13, wl.dtype)
            w2p[e], w2s[e] = p2, e8m0_to_h16(e2, wl.dtype)
            continue
        w13p[e], w13s[e] = quantize_matrix(w13, wl.per_channel, wl.dtype)
        w2p[e], w2s[e] = quantize_matrix(w2, wl.per_channel, wl.dtype)
    return Weights(w13p, w13s, w2p, w2s)


def make_weights_fp32(wl: Workload, device="cpu", seed: Optional[int] = None, std: float = 0.02):
    """The fp32 master weights that make_weights quantizes (for quantizer pins)."""
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed if seed is None else seed)
    out = []
    for _ in range(wl.num_experts):
        w13 = torch.randn(wl.n1, wl.hidden, generator=g, device=device) * std
        w2 = torch.randn(wl.hidden, wl.inter, generator=g, device=device) * std
        out.append((w13, w2))
    return out


# ---------------------------------------------------------------------------
# tokens and routes
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Tokens:
    x: torch.Tensor             # [T, H] 16-bit
    topk_ids: torch.Tensor      # [T, K] int32, global ids
    topk_weights: torch.Tensor  # [T, K] fp32
    skew_bias: float = 0.0
    hot_share: float = float("nan")
    logits: Optional[torch.Tensor] = None  # [T, E_global] fp32 the routes came from

    def to(self, device) -> "Tokens":
        return Tokens(self.x.to(device), self.topk_ids.to(device), self.topk_weights.to(device),
                      self.skew_bias, self.hot_share,
                      None if self.logits is None else self.logits.to(device))


def _route(logits: torch.Tensor, k: int):
    probs = torch.softmax(logits, dim=-1)
    w, ids = torch.topk(probs, k, dim=-1, largest=True, sorted=True)
    return ids.to(torch.int32).contiguous(), w.to(torch.float32).contiguous()


HOT_EXPERTS = (0, 1, 2, 3)


def _skew_logits(logits: torch.Tensor, b: float) -> torch.Tensor:
    """The skewed workload's effective router logits: experts e = 15 (mod 16)
    masked to -inf, the hot experts raised by b."""
    E = logits.shape[1]
    masked = torch.tensor([e % 16 == 15 for e in range(E)], device=logits.device)
    hot = torch.zeros(E, dtype=torch.bool, device=logits.device)
    hot[list(HOT_EXPERTS)] = True
    return logits.masked_fill(masked, float("-inf")) + b * hot.float()


def _skewed_route(logits: torch.Tensor, k: int, target: float = 0.25):
    E = logits.shape[1]
    masked = torch.tensor([e % 16 == 15 for e in range(E)], device=logits.device)
    hot = torch.zeros(E, dtype=torch.bool, device=logits.device)
    hot[list(HOT_EXPERTS)] = True
    base = logits.masked_fill(masked, float("-inf"))

    def share(b):
        ids, _ = _route(base + b * hot.float(), k)
        return hot[ids.long()].float().mean().item()

    lo, hi = 0.0, 16.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if share(mid) < target:
            lo = mid
        else:
            hi = mid
    b = lo if abs(share(lo) - target) <= abs(share(hi) - target) else hi
    ids, w = _route(base + b * hot.float(), k)
    return ids, w, b, share(b)


def make_tokens(wl: Workload, T: int, device="cpu", seed: Optional[int] = None) -> Tokens:
    g = torch.Generator(device=device)
    g.manual_seed((wl.seed if seed is None else seed) + T)
    x = torch.randn(T, wl.hidden, generator=g, device=device, dtype=torch.float32).to(wl.dtype)
    logits = torch.randn(T, wl.num_global_experts, generator=g, device=device,
                         dtype=torch.float32)
    if wl.skew and T > 0:
        ids, w, b, sh = _skewed_route(logits, wl.top_k)
        eff = _skew_logits(logits, b)
        return Tokens(x.contiguous(), ids, w, b, sh, eff.contiguous())
    ids, w = _route(logits, wl.top_k)
    return Tokens(x.contiguous(), ids, w, logits=logits.contiguous())
