"""GPU parity of the FP4-weight layout (E2M1 codes along K, a 16-bit scale per
32 values; MXFP4 scales converted exactly) through the C ABI against the CPU
oracle: the device E2M1 decode (the GEMMs' conversion) bit-exact against the
element format's table for every byte at every place in a dword, the E8M0
scale conversion bit-exact, the forward within the NRMSE
bar on every variant (small batch, streaming and split-K gate/up, resident
and streaming down, fused finalize), ragged reductions, both 16-bit types,
and the Kimi-shard and DeepSeek-share shapes at full size."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
from moe_check import assert_close, forward, oracle_out, tokens, weights
from w4a16_mixture_experts_amd import binding, synth

pytestmark = pytest.mark.gpu


def _e2m1_table():
    """The element format's 16 values (tests/golden/fp4_e2m1.txt)."""
    tab = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "fp4_e2m1.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                code, val = line.split()
                tab[int(code, 16)] = np.float32(float(val))
    assert sorted(tab) == list(range(16))
    return tab


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("n", [1024, 1027, 3])
def test_device_e2m1_decode_bit_exact(dtype, n):
    """Every byte value at each of the four byte places of a dword (the
    conversion pairs the codes of a dword four apart), a ragged tail, both
    16-bit types: the values and the signs of zero as the table gives them."""
    tab = _e2m1_table()
    b = np.concatenate([np.repeat(np.arange(256, dtype=np.uint8), 4),
                        np.array([0x8F, 0x07, 0xF8], np.uint8)])[:n]
    got = binding.decode_fp4(torch.from_numpy(b).cuda(), dtype)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = np.empty(2 * n, np.float32)
    want[0::2] = [tab[int(x) & 0xF] for x in b]
    want[1::2] = [tab[int(x) >> 4] for x in b]
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    np.testing.assert_array_equal(got, oracle.unpack_fp4(b))


def test_e8m0_conversion_bit_exact():
    e = torch.arange(256, dtype=torch.uint8)
    got = binding.e8m0_to_scales(e.cuda(), torch.bfloat16).cpu()
    want = oracle.e8m0_to_f32(e.numpy())
    np.testing.assert_array_equal(got[:255].float().numpy(), want[:255])
    assert torch.isnan(got[255].float())
    ok = torch.arange(103, 143, dtype=torch.uint8)      # the powers of two fp16 holds
    got16 = binding.e8m0_to_scales(ok.cuda(), torch.float16).cpu()
    np.testing.assert_array_equal(got16.float().numpy(), oracle.e8m0_to_f32(ok.numpy()))
    # the generator's 16-bit scales are these very values
    torch.testing.assert_close(synth.e8m0_to_h16(e[:255], torch.bfloat16), got[:255], rtol=0,
                               atol=0)


TINY_FP4 = dataclasses.replace(synth.WORKLOADS["tiny"], name="tiny_fp4", fp4=True)
VARIANTS = [dict(force_path=2), dict(force_path=1), dict(force_path=1, force_splitk=1),
            dict(force_path=1, force_splitk=2), dict(force_path=1, fused_finalize=1)]


@pytest.fixture(scope="module")
def tiny_fp4():
    Wc = synth.make_weights(TINY_FP4, device="cpu")
    return Wc, Wc.to("cuda")


@pytest.mark.parametrize("force", VARIANTS, ids=lambda f: "-".join(f"{k}{v}" for k, v in f.items()))
@pytest.mark.parametrize("T", [16, 256])
def test_tiny_fp4_all_variants(tiny_fp4, force, T):
    if T * TINY_FP4.top_k > 128 and force.get("force_path") == 2:
        pytest.skip("the small-batch path takes at most 128 routes")
    Wc, Wg = tiny_fp4
    tc = tokens(TINY_FP4, T)
    out = forward(TINY_FP4, Wg, tc.to("cuda"), **force)
    assert_close(out, oracle_out(TINY_FP4, Wc, tc), f"tiny fp4 T={T} {force}")


@pytest.mark.parametrize("gated,dtype", [(True, torch.bfloat16), (False, torch.float16)])
def test_fp4_ragged_tails_and_dtypes(gated, dtype):
    """H = 320, I = 192 (reductions ending in a half block), both 16-bit
    types, gated and ReLU^2, on every path."""
    wl = synth.custom("tails_fp4", E=4, H=320, I=192, K=2, gated=gated, dtype=dtype, fp4=True,
                      seed=7)
    Wc = synth.make_weights(wl, device="cpu")
    Wg = Wc.to("cuda")
    for T, force in ((150, dict(force_path=1, force_splitk=2)),
                     (150, dict(force_path=1, force_splitk=1)), (40, dict(force_path=1)),
                     (20, dict(force_path=2))):
        tc = tokens(wl, T)
        out = forward(wl, Wg, tc.to("cuda"), **force)
        assert_close(out, oracle_out(wl, Wc, tc), f"fp4 tails T={T} {force}")


def test_fp4_differs_from_int4_reading(tiny_fp4):
    """The same bytes read as INT4 give a different result: the layout field
    reaches the kernels."""
    Wc, Wg = tiny_fp4
    tg = tokens(TINY_FP4, 16, "cuda")
    a = forward(TINY_FP4, Wg, tg)
    b = forward(dataclasses.replace(TINY_FP4, fp4=False), Wg, tg)
    assert not torch.equal(a, b)


@pytest.mark.parametrize("name,T", [("kimi_tp8_fp4", 1), ("kimi_tp8_fp4", 8),
                                    ("kimi_tp8_fp4", 32), ("kimi_tp8_fp4", 256),
                                    ("deepseek_local_fp4", 1), ("deepseek_local_fp4", 16),
                                    ("deepseek_local_fp4", 128)])
def test_fp4_workloads_whole_output(name, T):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tc = tokens(wl, T)
    out = forward(wl, Wg, tc.to("cuda"))
    assert_close(out, oracle_out(wl, Wc, tc), f"{name} T={T}")


@pytest.mark.parametrize("name,T", [("kimi_tp8_fp4", 1024), ("kimi_tp8_fp4", 2048),
                                    ("deepseek_local_fp4", 512), ("deepseek_local_fp4", 2048)])
def test_fp4_workloads_sampled_rows(name, T):
    wl = synth.WORKLOADS[name]
    Wc, Wg = weights(name)
    tc = tokens(wl, T)
    out = forward(wl, Wg, tc.to("cuda"))
    rows = sorted(set([0, T - 1] + np.random.default_rng(T).choice(T, 30, replace=False).tolist()))
    ref = oracle_out(wl, Wc, tc, rows=rows)
    assert_close(out[torch.as_tensor(rows, device="cuda")], ref, f"{name} T={T} rows")
