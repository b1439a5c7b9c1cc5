"""Pins of the CPU oracle to things other than itself.

Each test fixes part of the oracle against mathematics or an independent
implementation: the page's packing rule on hand-written bytes, exact round
trips, closed-form outputs, a float64 numpy textbook FFN, a dense brute-force
evaluation of every expert, brute-force route tables and exact invariances.
A plausible slip anywhere in the oracle (a swapped nibble, gate/up order, a
dropped route, a wrong index or sign) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from w4a16_mixture_experts_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent helpers (numpy bit tricks, float64)
# ---------------------------------------------------------------------------

def np_unpack(b):
    """Sign-extend nibbles with arithmetic shifts (no branches, no table)."""
    b = np.asarray(b, np.uint8)
    lo = (b << 4).view(np.int8) >> 4
    hi = b.view(np.int8) >> 4
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def np_h16(bits, dtype):
    bits = np.asarray(bits, np.uint16)
    if dtype == oracle.DT_BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def np_dequant(packed, scales, layout, dtype, group=32):
    """fp64 dequantized [E, n_out, k_in] from packed weights, written independently."""
    packed = np.asarray(packed)
    s = np_h16(scales, dtype)
    if layout == oracle.Q_GROUP_K:
        q = np_unpack(packed).astype(np.float64)             # [E, n, k]
        E, n, k = q.shape
        return q * np.repeat(s, group, axis=2)
    # per-channel: packed [E, n/2, k] along n
    E, half, k = packed.shape
    lo = ((packed << 4).view(np.int8) >> 4).astype(np.float64)
    hi = (packed.view(np.int8) >> 4).astype(np.float64)
    q = np.empty((E, 2 * half, k))
    q[:, 0::2, :] = lo
    q[:, 1::2, :] = hi
    return q * s[:, :, None]


def np_ffn(x, w13, w2, gated):
    h = x @ w13.T
    if gated:
        I = w13.shape[0] // 2
        g, u = h[..., :I], h[..., I:]
        a = g / (1.0 + np.exp(-g)) * u
    else:
        a = np.maximum(h, 0.0) ** 2
    return a @ w2.T


def bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def run_oracle(wl, W, tok, **kw):
    return oracle.moe_forward(
        bits(tok.x), W.w13_packed.numpy(), bits(W.w13_scales), W.w2_packed.numpy(),
        bits(W.w2_scales), tok.topk_ids.numpy(), tok.topk_weights.numpy(), hidden=wl.hidden,
        inter=wl.inter, num_experts=wl.num_experts, expert_offset=wl.expert_offset,
        act=oracle.ACT_SILU_GATED if wl.gated else oracle.ACT_RELU2,
        layout=oracle.Q_PER_CHANNEL if wl.per_channel else oracle.Q_GROUP_K,
        dtype=oracle.DT_FP16 if wl.dtype == torch.float16 else oracle.DT_BF16, **kw)


def dt_code(wl):
    return oracle.DT_FP16 if wl.dtype == torch.float16 else oracle.DT_BF16


# ---------------------------------------------------------------------------
# 16-bit conversions against numpy / torch
# ---------------------------------------------------------------------------

SPECIALS = np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.0, 65520.0, 1e30, -1e30, np.inf,
                     -np.inf, 6.1e-5, 5.96e-8, 2.98e-8, 2.99e-8, 1e-40, 3.0e38, 1.00390625,
                     1.0078125, 1.01171875, 0.1, 1.0 / 3.0], np.float32)


@pytest.mark.parametrize("dtype", [oracle.DT_BF16, oracle.DT_FP16])
def test_h16_conversions_match_numpy_and_torch(dtype):
    rng = np.random.default_rng(1)
    x = np.concatenate([SPECIALS, rng.standard_normal(20000).astype(np.float32) * 10,
                        (rng.standard_normal(5000) * 1e-6).astype(np.float32)])
    got = oracle.f32_to_h16(x, dtype)
    if dtype == oracle.DT_FP16:
        want = x.astype(np.float16).view(np.uint16)
    else:
        want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    # every 16-bit pattern back to fp32 (NaNs compared as NaN)
    allbits = np.arange(65536, dtype=np.uint16)
    back = oracle.h16_to_f32(allbits, dtype)
    ref = np_h16(allbits, dtype).astype(np.float32)
    np.testing.assert_array_equal(np.isnan(back), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(back[ok].view(np.uint32), ref[ok].view(np.uint32))


# ---------------------------------------------------------------------------
# packing (page rule, exhaustive)
# ---------------------------------------------------------------------------

def test_nibble_fixture():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "nibbles.txt"))
            if ln.strip() and not ln.startswith("#")]
    b = np.array([int(r[0], 16) for r in rows], np.uint8)
    want = np.array([[int(r[1]), int(r[2])] for r in rows], np.int8).reshape(-1)
    np.testing.assert_array_equal(oracle.unpack_int4(b), want)
    np.testing.assert_array_equal(oracle.pack_int4(want), b)


def test_nibbles_exhaustive_and_round_trip():
    b = np.arange(256, dtype=np.uint8)
    q = oracle.unpack_int4(b)
    np.testing.assert_array_equal(q, np_unpack(b))
    assert q.min() == -8 and q.max() == 7
    np.testing.assert_array_equal(oracle.pack_int4(q), b)
    pairs = np.array([[lo, hi] for lo in range(-8, 8) for hi in range(-8, 8)], np.int8).ravel()
    np.testing.assert_array_equal(oracle.unpack_int4(oracle.pack_int4(pairs)), pairs)


# ---------------------------------------------------------------------------
# quantizer: exact round trip, an exact-rational example, the generator
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [oracle.DT_BF16, oracle.DT_FP16])
def test_quantize_dequant_round_trip(dtype):
    rng = np.random.default_rng(2)
    rows, cols = 16, 128
    q = rng.integers(-7, 8, size=(rows, cols)).astype(np.int8)
    q[:, ::32] = rng.choice([-7, 7], size=(rows, cols // 32))      # every group hits |q| = 7
    s = oracle.f32_to_h16(np.exp(rng.uniform(-9, -2, size=(rows, cols // 32))), dtype)
    w = q.astype(np.float32) * np.repeat(oracle.h16_to_f32(s, dtype), 32, axis=1)
    q2, s2 = oracle.quantize_group(w, 32, dtype)
    np.testing.assert_array_equal(s2, s)
    np.testing.assert_array_equal(q2, q)
    # per-channel: one |q| = 7 per row
    qc = rng.integers(-7, 8, size=(rows, cols)).astype(np.int8)
    qc[:, 5] = 7
    sc = oracle.f32_to_h16(np.exp(rng.uniform(-9, -2, size=rows)), dtype)
    wc = qc.astype(np.float32) * oracle.h16_to_f32(sc, dtype)[:, None]
    q3, s3 = oracle.quantize_per_channel(wc, dtype)
    np.testing.assert_array_equal(s3, sc)
    np.testing.assert_array_equal(q3, qc)


def test_quantize_exact_rational_example():
    """scale = absmax/7 rounded to bf16; q = nearest (ties to even) of w/scale."""
    from fractions import Fraction as F
    w = np.zeros((1, 32), np.float32)
    w[0, :6] = [0.7, -0.35, 0.05, -0.7, 0.3, 0.0]
    q, s = oracle.quantize_group(w, 32, oracle.DT_BF16)
    sv = float(np_h16(s, oracle.DT_BF16)[0, 0])
    # bf16 of 0.1 (0.7/7 in fp32) is 0.10009765625 = 205 * 2^-11
    assert sv == 205 * 2.0 ** -11
    want = []
    for v in w[0]:
        r = F(float(v)) / F(sv)
        fl = math.floor(r)
        frac = r - fl
        n = fl + (1 if frac > F(1, 2) or (frac == F(1, 2) and fl % 2 == 1) else 0)
        want.append(max(-8, min(7, n)))
    np.testing.assert_array_equal(q[0], np.array(want, np.int8))
    assert list(q[0, :6]) == [7, -3, 0, -7, 3, 0]
    # an all-zero group has scale 0 and codes 0
    qz, sz = oracle.quantize_group(np.zeros((2, 64), np.float32), 32, oracle.DT_BF16)
    assert not qz.any() and not sz.any()


@pytest.mark.parametrize("per_channel,dtype", [(False, torch.bfloat16), (True, torch.bfloat16),
                                               (False, torch.float16), (True, torch.float16)])
def test_generator_quantizer_equals_oracle(per_channel, dtype):
    wl = synth.custom(E=2, H=64, I=96, K=2, per_channel=per_channel, dtype=dtype, seed=5)
    W = synth.make_weights(wl)
    masters = synth.make_weights_fp32(wl)
    dt = dt_code(wl)
    for e, (w13, w2) in enumerate(masters):
        for w, packed, sc in ((w13, W.w13_packed[e], W.w13_scales[e]),
                              (w2, W.w2_packed[e], W.w2_scales[e])):
            if per_channel:
                q, s = oracle.quantize_per_channel(w.numpy(), dt)
                want_packed = oracle.pack_int4(q.T.copy()).T       # pairs of rows
            else:
                q, s = oracle.quantize_group(w.numpy(), 32, dt)
                want_packed = oracle.pack_int4(q)
            np.testing.assert_array_equal(bits(sc), s)
            np.testing.assert_array_equal(packed.numpy(), want_packed)


@pytest.mark.parametrize("layout", [oracle.Q_GROUP_K, oracle.Q_PER_CHANNEL])
def test_dequant_matrix_matches_numpy(layout):
    wl = synth.custom(E=1, H=64, I=96, K=1, per_channel=layout == oracle.Q_PER_CHANNEL, seed=3)
    W = synth.make_weights(wl)
    got = oracle.dequant_matrix(W.w13_packed[0].numpy(), bits(W.w13_scales[0]), 2 * 96, 64,
                                layout, 32, oracle.DT_BF16)
    want = np_dequant(W.w13_packed.numpy(), bits(W.w13_scales), layout, oracle.DT_BF16)[0]
    np.testing.assert_array_equal(got.astype(np.float64), want)       # q*s exact in fp32


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _golden_closed_form():
    vals = {}
    for ln in open(os.path.join(GOLDEN, "closed_form.txt")):
        ln = ln.split("#")[0].strip()
        if ln:
            k, v = ln.split()[:2]
            vals[k] = float(v)
    return vals


def _bf16_bits(v):
    return int(torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).view(torch.int16)) & 0xFFFF


def _closed_form_case(per_channel, gated=True, x_val=1.0, K=1, wts=(1.0,)):
    E, H, I = 1, 64, 32
    N1 = 2 * I if gated else I
    q13 = np.ones((N1, H), np.int8)
    if gated:
        q13[I:] = 2
    q2 = np.ones((H, I), np.int8)
    s6, s5 = _bf16_bits(2.0 ** -6), _bf16_bits(2.0 ** -5)
    if per_channel:
        w13p = oracle.pack_int4(q13.T.copy()).T[None].copy()
        w2p = oracle.pack_int4(q2.T.copy()).T[None].copy()
        w13s = np.full((1, N1), s6, np.uint16)
        w2s = np.full((1, H), s5, np.uint16)
    else:
        w13p = oracle.pack_int4(q13)[None]
        w2p = oracle.pack_int4(q2)[None]
        w13s = np.full((1, N1, H // 32), s6, np.uint16)
        w2s = np.full((1, H, I // 32), s5, np.uint16)
    x = np.full((1, H), _bf16_bits(x_val), np.uint16)
    ids = np.zeros((1, K), np.int32)
    w = np.array([wts], np.float32)
    return oracle.moe_forward(x, w13p, w13s, w2p, w2s, ids, w, hidden=H, inter=I, num_experts=E,
                              act=oracle.ACT_SILU_GATED if gated else oracle.ACT_RELU2,
                              layout=oracle.Q_PER_CHANNEL if per_channel else oracle.Q_GROUP_K)


@pytest.mark.parametrize("per_channel", [False, True])
def test_closed_form(per_channel):
    g = _golden_closed_form()
    out = _closed_form_case(per_channel)
    assert out.shape == (1, 64)
    np.testing.assert_allclose(out, g["gated_out"], rtol=1e-6)
    assert abs(out[0, 0] - g["gated_out_swapped"]) > 0.1          # gate rows come first
    assert _bf16_bits(float(out[0, 0])) == _bf16_bits(g["gated_out_bf16"])
    np.testing.assert_allclose(_closed_form_case(per_channel, gated=False), g["relu2_out_x_pos"],
                               rtol=0)
    np.testing.assert_array_equal(_closed_form_case(per_channel, gated=False, x_val=-1.0),
                                  g["relu2_out_x_neg"])
    dup = _closed_form_case(per_channel, K=2, wts=(0.25, 0.5))
    np.testing.assert_allclose(dup, g["dup_routes_0.25_0.5"], rtol=1e-6)


# ---------------------------------------------------------------------------
# textbook FFN and dense brute force (float64 numpy)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("per_channel,gated,dtype", [
    (False, True, torch.bfloat16), (True, True, torch.bfloat16),
    (False, False, torch.float16), (True, False, torch.float16)])
def test_single_expert_equals_textbook_ffn(per_channel, gated, dtype):
    wl = synth.custom(E=3, H=128, I=64, K=1, gated=gated, per_channel=per_channel, dtype=dtype,
                      seed=11)
    W = synth.make_weights(wl)
    tok = synth.make_tokens(wl, 5)
    tok.topk_ids[:] = 1
    tok.topk_weights[:] = 1.0
    out = run_oracle(wl, W, tok)
    lay = oracle.Q_PER_CHANNEL if per_channel else oracle.Q_GROUP_K
    dt = dt_code(wl)
    w13 = np_dequant(W.w13_packed.numpy(), bits(W.w13_scales), lay, dt)[1]
    w2 = np_dequant(W.w2_packed.numpy(), bits(W.w2_scales), lay, dt)[1]
    x = np_h16(bits(tok.x), dt)
    want = np_ffn(x, w13, w2, gated)
    np.testing.assert_allclose(out, want, rtol=1e-4, atol=1e-5 * np.abs(want).max())


@pytest.mark.parametrize("per_channel,gated,offset,E_global", [
    (False, True, 0, 6), (True, True, 0, 6), (False, False, 0, 6), (False, True, 4, 16)])
def test_brute_force_dense_all_experts(per_channel, gated, offset, E_global):
    E, H, I, K, T = 6, 64, 96, 3, 7
    wl = synth.custom(E=E, H=H, I=I, K=K, gated=gated, per_channel=per_channel, seed=23,
                      E_global=E_global, offset=offset)
    W = synth.make_weights(wl)
    tok = synth.make_tokens(wl, T)
    ids = tok.topk_ids.numpy()
    # plant invalid ids: negative, past the end, and (with an offset) below it
    ids[0, 1] = -1
    ids[2, 0] = offset + E + 3
    ids[3, :] = -7                                            # a token without a valid route
    out = run_oracle(wl, W, tok)
    lay = oracle.Q_PER_CHANNEL if per_channel else oracle.Q_GROUP_K
    w13 = np_dequant(W.w13_packed.numpy(), bits(W.w13_scales), lay, oracle.DT_BF16)
    w2 = np_dequant(W.w2_packed.numpy(), bits(W.w2_scales), lay, oracle.DT_BF16)
    x = np_h16(bits(tok.x), oracle.DT_BF16)
    Y = np.stack([np_ffn(x, w13[e], w2[e], gated) for e in range(E)], axis=1)   # [T, E, H]
    M = np.zeros((T, E))
    for t in range(T):
        for k in range(K):
            e = ids[t, k] - offset
            if 0 <= e < E:
                M[t, e] += tok.topk_weights[t, k].item()
    want = np.einsum("te,teh->th", M, Y)
    scale = np.abs(want).max()
    np.testing.assert_allclose(out, want, rtol=1e-4, atol=1e-5 * scale)
    assert not out[3].any() and not np.signbit(out[3]).any()        # exactly +0


def test_per_route_outputs_match_brute_force():
    E, H, I, K, T = 4, 64, 64, 2, 5
    wl = synth.custom(E=E, H=H, I=I, K=K, seed=31)
    W = synth.make_weights(wl)
    tok = synth.make_tokens(wl, T)
    tok.topk_ids[1, 1] = 99
    out, yr = run_oracle(wl, W, tok, want_routes=True)
    w13 = np_dequant(W.w13_packed.numpy(), bits(W.w13_scales), oracle.Q_GROUP_K, oracle.DT_BF16)
    w2 = np_dequant(W.w2_packed.numpy(), bits(W.w2_scales), oracle.Q_GROUP_K, oracle.DT_BF16)
    x = np_h16(bits(tok.x), oracle.DT_BF16)
    for t in range(T):
        for k in range(K):
            e = int(tok.topk_ids[t, k])
            r = t * K + k
            if e >= E:
                assert np.isnan(yr[r]).all()                       # never written
                continue
            want = np_ffn(x[t], w13[e], w2[e], True)
            np.testing.assert_allclose(yr[r], want, rtol=1e-4, atol=1e-5 * np.abs(want).max())


# ---------------------------------------------------------------------------
# exact invariances
# ---------------------------------------------------------------------------

def test_invariances_bitwise():
    E, H, I, K, T = 5, 64, 64, 3, 9
    wl = synth.custom(E=E, H=H, I=I, K=K, seed=41)
    W = synth.make_weights(wl)
    tok = synth.make_tokens(wl, T)
    base = run_oracle(wl, W, tok)
    # (i) weights x2 -> output x2 exactly
    tok2 = synth.Tokens(tok.x, tok.topk_ids, tok.topk_weights * 2)
    np.testing.assert_array_equal(run_oracle(wl, W, tok2), base * 2)
    # (ii) token permutation -> output permutation exactly
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(0))
    tokp = synth.Tokens(tok.x[perm].contiguous(), tok.topk_ids[perm].contiguous(),
                        tok.topk_weights[perm].contiguous())
    np.testing.assert_array_equal(run_oracle(wl, W, tokp), base[perm.numpy()])
    # (iii) one invalid id for another -> same bits; all invalid -> zeros
    ids_a = tok.topk_ids.clone()
    ids_a[2, 1] = -3
    ids_b = tok.topk_ids.clone()
    ids_b[2, 1] = 1000
    oa = run_oracle(wl, W, synth.Tokens(tok.x, ids_a, tok.topk_weights))
    ob = run_oracle(wl, W, synth.Tokens(tok.x, ids_b, tok.topk_weights))
    np.testing.assert_array_equal(oa, ob)
    assert not np.array_equal(oa, base)
    allbad = torch.full_like(tok.topk_ids, E)
    np.testing.assert_array_equal(run_oracle(wl, W, synth.Tokens(tok.x, allbad,
                                                                 tok.topk_weights)), 0.0)
    # (iv) relabel experts consistently -> same bits
    pe = torch.tensor([3, 0, 4, 1, 2])                     # new id of old expert e
    inv = torch.argsort(pe)
    Wr = synth.Weights(W.w13_packed[inv].contiguous(), W.w13_scales[inv].contiguous(),
                       W.w2_packed[inv].contiguous(), W.w2_scales[inv].contiguous())
    ids_r = pe[tok.topk_ids.long()].to(torch.int32)
    np.testing.assert_array_equal(run_oracle(wl, Wr, synth.Tokens(tok.x, ids_r,
                                                                  tok.topk_weights)), base)


def test_empty_batch():
    wl = synth.custom(E=2, H=64, I=32, K=2)
    W = synth.make_weights(wl)
    tok = synth.make_tokens(wl, 0)
    assert run_oracle(wl, W, tok).shape == (0, 64)


# ---------------------------------------------------------------------------
# route tables against brute force
# ---------------------------------------------------------------------------

def brute_routes(ids, E, off, bm):
    T, K = ids.shape
    flat = ids.reshape(-1)
    per = [[r for r in range(T * K) if flat[r] - off == e] for e in range(E)]
    counts = [len(p) for p in per]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + -(-c // bm) * bm)
    srt = [-1] * offsets[-1]
    slot = [-1] * (T * K)
    for e, p in enumerate(per):
        for j, r in enumerate(p):
            srt[offsets[e] + j] = r
            slot[r] = offsets[e] + j
    return counts, offsets, srt, slot


@pytest.mark.parametrize("T,K,E,E_global,off,bm", [
    (16, 2, 8, 8, 0, 16), (7, 3, 5, 9, 2, 4), (1, 8, 384, 384, 0, 16), (33, 6, 128, 128, 0, 64),
    (0, 4, 8, 8, 0, 16), (50, 8, 32, 256, 0, 32), (40, 8, 32, 256, 96, 1)])
def test_prepare_routes_brute_force(T, K, E, E_global, off, bm):
    rng = np.random.default_rng(T * 1000 + K)
    ids = rng.integers(-2, E_global + 2, size=(T, K)).astype(np.int32)
    counts, offsets, srt, slot = oracle.prepare_routes(ids, E, off, bm)
    bc, bo, bs, bsl = brute_routes(ids, E, off, bm)
    assert counts.tolist() == bc and offsets.tolist() == bo
    assert srt.tolist() == bs and slot.tolist() == bsl
    # invariants: padded offsets are multiples of bm; slot inverts sorted
    assert all(o % bm == 0 for o in offsets)
    for r, p in enumerate(slot):
        if p >= 0:
            assert srt[p] == r


# ---------------------------------------------------------------------------
# router scoring and top-k (softmax over all global experts, K largest)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,Eg,K", [(5, 8, 2), (7, 256, 8), (3, 384, 8), (4, 1024, 32)])
def test_route_topk_matches_float64_softmax_topk(T, Eg, K):
    """Random N(0,1) logits (no ties): same ids and order as torch's float64
    softmax followed by topk, weights equal to the float64 probabilities."""
    rng = np.random.default_rng(Eg + K)
    logits = rng.standard_normal((T, Eg)).astype(np.float32)
    ids, w = oracle.route_topk(logits, K)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=-1)
    ref_w, ref_i = torch.topk(p, K, dim=-1)
    np.testing.assert_array_equal(ids, ref_i.numpy())
    np.testing.assert_allclose(w, ref_w.numpy(), rtol=1e-6, atol=0)


def test_route_topk_closed_forms():
    # probabilities 1/6, 2/6, 3/6: the two largest are experts 2 and 1
    logits = np.log(np.array([[1.0, 2.0, 3.0]], np.float64)).astype(np.float32)
    ids, w = oracle.route_topk(logits, 2)
    np.testing.assert_array_equal(ids, [[2, 1]])
    np.testing.assert_allclose(w, [[0.5, 1.0 / 3.0]], rtol=1e-6)
    # equal logits: every probability 1/E, ids in ascending order
    ids, w = oracle.route_topk(np.zeros((2, 12), np.float32), 5)
    np.testing.assert_array_equal(ids, [[0, 1, 2, 3, 4]] * 2)
    np.testing.assert_array_equal(w, np.full((2, 5), np.float32(1.0 / 12.0)))
    # ties go to the lower id
    ids, w = oracle.route_topk(np.array([[1, 3, 3, 2, 3]], np.float32), 4)
    np.testing.assert_array_equal(ids, [[1, 2, 4, 3]])
    assert w[0, 0] == w[0, 1] == w[0, 2] > w[0, 3]


def test_route_topk_masked_experts_and_renormalization():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((6, 64)).astype(np.float32)
    logits[:, 15::16] = -np.inf                   # masked experts never chosen
    ids, w = oracle.route_topk(logits, 6)
    assert not np.isin(ids, np.arange(15, 64, 16)).any()
    p = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids, 1), rtol=1e-6)
    # renormalized: same ids, weights proportional, summing to 1
    ids_r, w_r = oracle.route_topk(logits, 6, renormalize=True)
    np.testing.assert_array_equal(ids_r, ids)
    np.testing.assert_allclose(w_r.sum(axis=1), 1.0, rtol=1e-6)
    np.testing.assert_allclose(w_r, w / w.sum(axis=1, keepdims=True), rtol=1e-6)
    # a token whose logits are all -inf: zero weights, lowest ids
    ids_m, w_m = oracle.route_topk(np.full((1, 8), -np.inf, np.float32), 3)
    np.testing.assert_array_equal(ids_m, [[0, 1, 2]])
    np.testing.assert_array_equal(w_m, np.zeros((1, 3), np.float32))


def test_route_topk_shift_invariance():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((9, 384)).astype(np.float32)
    ids, w = oracle.route_topk(logits, 8)
    ids2, w2 = oracle.route_topk(logits + np.float32(4.0), 8)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-5)


# ---------------------------------------------------------------------------
# FP4 (MXFP4: E2M1 codes, E8M0 block scales) weights
# ---------------------------------------------------------------------------

def _golden_table(name, conv):
    out = []
    for ln in open(os.path.join(GOLDEN, name)):
        ln = ln.split("#")[0].strip()
        if ln:
            a, b = ln.split()[:2]
            out.append(conv(a, b))
    return out


def _e2m1_golden():
    tab = dict(_golden_table("fp4_e2m1.txt", lambda a, b: (int(a, 16), float(b))))
    assert sorted(tab) == list(range(16))
    return np.array([tab[c] for c in range(16)], np.float64)


def np_dequant_fp4(packed, scales, dtype):
    """fp64 [E, n, k] from E2M1 codes through the fixture's value table."""
    tab = _e2m1_golden()
    packed = np.asarray(packed, np.uint8)
    codes = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.int64)
    codes[..., 0::2] = packed & 0xF
    codes[..., 1::2] = packed >> 4
    return tab[codes] * np.repeat(np_h16(scales, dtype), 32, axis=-1)


def test_fp4_code_table_exhaustive():
    """Every byte: low nibble -> the even value, high nibble -> the odd one,
    against the OCP value table of the fixture; signs of zero included."""
    tab = _e2m1_golden()
    b = np.arange(256, dtype=np.uint8)
    got = oracle.unpack_fp4(b)
    np.testing.assert_array_equal(got[0::2], tab[b & 0xF])
    np.testing.assert_array_equal(got[1::2], tab[b >> 4])
    np.testing.assert_array_equal(np.signbit(got[0::2]), (b & 0x8) != 0)
    # the eight magnitudes, and symmetry
    assert sorted(set(np.abs(tab).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    np.testing.assert_array_equal(tab[8:], -tab[:8])


def test_e8m0_decode_every_code():
    e = np.arange(256, dtype=np.uint8)
    got = oracle.e8m0_to_f32(e).astype(np.float64)
    np.testing.assert_array_equal(got[:255], np.ldexp(1.0, e[:255].astype(np.int64) - 127))
    assert np.isnan(got[255])


def test_mxfp4_ties_fixture():
    cases = _golden_table("mxfp4_ties.txt", lambda a, b: (float(a), int(b, 16)))
    block = np.zeros(32, np.float32)
    block[:len(cases)] = [v for v, _ in cases]
    packed, sc = oracle.quantize_mxfp4(block[None])
    assert sc[0, 0] == 127
    codes = np.empty(32, np.int64)
    codes[0::2], codes[1::2] = packed[0] & 0xF, packed[0] >> 4
    for i, (v, want) in enumerate(cases):
        assert codes[i] == want, (v, codes[i], want)
    assert not codes[len(cases):].any()


def test_mxfp4_round_trip_and_exponent():
    """Blocks whose largest magnitude code is 4 or 6 keep their exponent:
    quantize(code value * 2^x) gives back the codes and E8M0 x + 127, for
    exponents across the E8M0 range that fp32 holds exactly."""
    rng = np.random.default_rng(5)
    tab = _e2m1_golden()
    for x in (-120, -40, -7, 0, 3, 60, 120):
        codes = rng.integers(0, 16, size=(8, 32))
        codes[:, 0] = rng.choice([0x6, 0x7, 0xE, 0xF], size=8)   # a magnitude 4 or 6
        w = (tab[codes] * 2.0 ** x).astype(np.float32)
        packed, sc = oracle.quantize_mxfp4(w)
        assert (sc == x + 127).all()
        got = np.empty_like(codes)
        got[:, 0::2], got[:, 1::2] = packed & 0xF, packed >> 4
        np.testing.assert_array_equal(got, codes)
    # an all-zero block: code 0 everywhere, E8M0 0
    packed, sc = oracle.quantize_mxfp4(np.zeros((1, 64), np.float32))
    assert not packed.any() and not sc.any()


def test_generator_mxfp4_equals_oracle():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((48, 320)) * 0.02).astype(np.float32)
    w[3, :32] = 0.0                                          # a zero block
    w[4, 40] = 1e-3 * 2.0 ** -60                             # a block of tiny values
    p, e = synth.quantize_mxfp4(torch.from_numpy(w))
    po, eo = oracle.quantize_mxfp4(w)
    np.testing.assert_array_equal(p.numpy(), po)
    np.testing.assert_array_equal(e.numpy(), eo)
    # the 16-bit scales are the exact powers of two
    s16 = synth.e8m0_to_h16(torch.from_numpy(eo), torch.bfloat16)
    np.testing.assert_array_equal(s16.float().numpy(), oracle.e8m0_to_f32(eo))


def test_fp4_dequant_matrix_matches_numpy():
    wl = synth.custom(E=1, H=64, I=96, K=1, fp4=True, seed=3)
    W = synth.make_weights(wl)
    got = oracle.dequant_matrix(W.w13_packed[0].numpy(), bits(W.w13_scales[0]), 2 * 96, 64,
                                oracle.Q_FP4_GROUP_K, 32, oracle.DT_BF16)
    want = np_dequant_fp4(W.w13_packed.numpy(), bits(W.w13_scales), oracle.DT_BF16)[0]
    np.testing.assert_array_equal(got.astype(np.float64), want)        # exact in fp32


def _fp4_closed_form(gated=True):
    """As the INT4 closed form: gate weights 1.0 (code 0x2), up 2.0 (0x4),
    down 1.0, scales 2^-6 and 2^-5, x = 1, H = 64, I = 32."""
    H, I = 64, 32
    N1 = 2 * I if gated else I
    c13 = np.full((N1, H), 0x2, np.uint8)
    if gated:
        c13[I:] = 0x4
    c2 = np.full((H, I), 0x2, np.uint8)
    w13p = (c13[:, 0::2] | (c13[:, 1::2] << 4))[None].copy()
    w2p = (c2[:, 0::2] | (c2[:, 1::2] << 4))[None].copy()
    w13s = np.full((1, N1, H // 32), _bf16_bits(2.0 ** -6), np.uint16)
    w2s = np.full((1, H, I // 32), _bf16_bits(2.0 ** -5), np.uint16)
    x = np.full((1, H), _bf16_bits(1.0), np.uint16)
    return oracle.moe_forward(x, w13p, w13s, w2p, w2s, np.zeros((1, 1), np.int32),
                              np.ones((1, 1), np.float32), hidden=H, inter=I, num_experts=1,
                              act=oracle.ACT_SILU_GATED if gated else oracle.ACT_RELU2,
                              layout=oracle.Q_FP4_GROUP_K)


def test_fp4_closed_form():
    g = _golden_closed_form()
    np.testing.assert_allclose(_fp4_closed_form(), g["gated_out"], rtol=1e-6)
    np.testing.assert_allclose(_fp4_closed_form(gated=False), g["relu2_out_x_pos"], rtol=0)


@pytest.mark.parametrize("gated,dtype", [(True, torch.bfloat16), (False, torch.float16)])
def test_fp4_brute_force_dense_all_experts(gated, dtype):
    E, H, I, K, T = 5, 64, 96, 2, 6
    wl = synth.custom(E=E, H=H, I=I, K=K, gated=gated, dtype=dtype, fp4=True, seed=29)
    W = synth.make_weights(wl)
    tok = synth.make_tokens(wl, T)
    ids = tok.topk_ids.numpy()
    ids[1, 0] = E + 2                                          # an invalid route
    dt = dt_code(wl)
    out = oracle.moe_forward(
        bits(tok.x), W.w13_packed.numpy(), bits(W.w13_scales), W.w2_packed.numpy(),
        bits(W.w2_scales), ids, tok.topk_weights.numpy(), hidden=H, inter=I, num_experts=E,
        act=oracle.ACT_SILU_GATED if gated else oracle.ACT_RELU2, layout=oracle.Q_FP4_GROUP_K,
        dtype=dt)
    w13 = np_dequant_fp4(W.w13_packed.numpy(), bits(W.w13_scales), dt)
    w2 = np_dequant_fp4(W.w2_packed.numpy(), bits(W.w2_scales), dt)
    x = np_h16(bits(tok.x), dt)
    Y = np.stack([np_ffn(x, w13[e], w2[e], gated) for e in range(E)], axis=1)
    M = np.zeros((T, E))
    for t in range(T):
        for k in range(K):
            if 0 <= ids[t, k] < E:
                M[t, ids[t, k]] += tok.topk_weights[t, k].item()
    want = np.einsum("te,teh->th", M, Y)
    np.testing.assert_allclose(out, want, rtol=1e-4, atol=1e-5 * np.abs(want).max())


# ---------------------------------------------------------------------------
# setup-only re-layout of per-channel weights into the group layout
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gated", [True, False])
def test_repack_per_channel_preserves_every_weight(gated):
    """The repacked group-layout weights dequantize (numpy float64, written
    independently) to exactly the per-channel weights, and the forward on
    them equals the per-channel forward bit for bit (same products, same
    ascending sums)."""
    wl = synth.custom(E=3, H=128, I=96, K=2, gated=gated, per_channel=True, seed=13)
    W = synth.make_weights(wl)
    p13, s13 = oracle.repack_per_channel(W.w13_packed.numpy(), bits(W.w13_scales))
    p2, s2 = oracle.repack_per_channel(W.w2_packed.numpy(), bits(W.w2_scales))
    np.testing.assert_array_equal(
        np_dequant(p13, s13, oracle.Q_GROUP_K, oracle.DT_BF16),
        np_dequant(W.w13_packed.numpy(), bits(W.w13_scales), oracle.Q_PER_CHANNEL, oracle.DT_BF16))
    np.testing.assert_array_equal(
        np_dequant(p2, s2, oracle.Q_GROUP_K, oracle.DT_BF16),
        np_dequant(W.w2_packed.numpy(), bits(W.w2_scales), oracle.Q_PER_CHANNEL, oracle.DT_BF16))
    tok = synth.make_tokens(wl, 9)
    a = run_oracle(wl, W, tok)
    b = oracle.moe_forward(bits(tok.x), p13, s13, p2, s2, tok.topk_ids.numpy(),
                           tok.topk_weights.numpy(), hidden=wl.hidden, inter=wl.inter,
                           num_experts=wl.num_experts,
                           act=oracle.ACT_SILU_GATED if gated else oracle.ACT_RELU2,
                           layout=oracle.Q_GROUP_K)
    np.testing.assert_array_equal(a, b)
    # a hand-checked byte: channels 0 and 1 of k = 0, 1 packed along N as
    # 0x9F (k=0: ch0 = -1, ch1 = -7) and 0x70 (k=1: ch0 = 0, ch1 = 7) become
    # along K ch0: (-1, 0) -> 0x0F, ch1: (-7, 7) -> 0x79
    pk = np.zeros((1, 1, 64), np.uint8)
    pk[0, 0, 0], pk[0, 0, 1] = 0x9F, 0x70
    rp, rs = oracle.repack_per_channel(pk, np.array([[0x3F80, 0x4000]], np.uint16))
    assert rp[0, 0, 0] == 0x0F and rp[0, 1, 0] == 0x79
    assert (rs[0, 0] == 0x3F80).all() and (rs[0, 1] == 0x4000).all()
