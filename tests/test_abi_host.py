"""Host-side tests of the C ABI: the library loads, exports every declared
entry point, and rejects malformed calls before anything reaches a GPU
(strict errors that name the offending tensor or field)."""
import ctypes
import os
import re

import pytest
import torch

from w4a16_mixture_experts_amd import binding as B
from w4a16_mixture_experts_amd import synth as S

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "w4a16_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = declared_functions()
    assert {"w4a16_moe_forward", "w4a16_moe_workspace_size", "w4a16_moe_prepare_routes",
            "w4a16_unpack_int4", "w4a16_status_string", "w4a16_last_error_message",
            "w4a16_moe_get_plan"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = B.lib()
    assert L.w4a16_status_string(0) == b"ok"
    assert L.w4a16_status_string(3) == b"workspace too small"
    assert L.w4a16_status_string(99) == b"unknown status"


def good(**kw):
    d = dict(num_tokens=4, hidden=256, intermediate=384, num_local_experts=8, top_k=2)
    d.update(kw)
    return B.make_desc(**d)


@pytest.mark.parametrize("field,value,status,needle", [
    ("num_tokens", -1, 1, "num_tokens"),
    ("hidden", 0, 1, "hidden"),
    ("intermediate", -64, 1, "intermediate"),
    ("num_local_experts", 0, 1, "num_local_experts"),
    ("top_k", 0, 1, "top_k"),
    ("dtype", 7, 1, "dtype"),
    ("act", 3, 1, "act"),
    ("qlayout", 3, 1, "qlayout"),
    ("num_local_experts", 2000, 2, "num_local_experts"),
    ("top_k", 33, 2, "top_k"),
    ("group_size", 64, 2, "group_size"),
    ("hidden", 96, 2, "hidden=96"),
    ("intermediate", 1828, 2, "intermediate=1828"),
    ("force_block_m", 48, 1, "force_block_m"),
    ("force_path", 3, 1, "force_path"),
    ("force_splitk", 3, 1, "force_splitk"),
    ("num_global_experts", 7, 1, "num_global_experts"),
    ("force_block_m", 32, 1, "force_block_m"),
    ("fp16_route", 2, 1, "fp16_route"),
])
def test_descriptor_errors(field, value, status, needle):
    d = good()
    setattr(d, field, value)
    n = ctypes.c_size_t(0)
    st = B.lib().w4a16_moe_workspace_size(ctypes.byref(d), ctypes.byref(n))
    assert st == status
    assert needle in B.lib().w4a16_last_error_message().decode()
    with pytest.raises(B.W4A16Error) as ei:
        B.workspace_size(d)
    assert ei.value.status == status


def test_null_descriptor():
    n = ctypes.c_size_t(0)
    assert B.lib().w4a16_moe_workspace_size(None, ctypes.byref(n)) == 1
    assert b"desc" in B.lib().w4a16_last_error_message()


def test_forward_rejects_before_launch():
    L = B.lib()
    d = good()
    need = B.workspace_size(d)
    P = ctypes.c_void_p
    fake = [P(0x10000 * (i + 1)) for i in range(8)]
    ws = P(0x900000)
    # null pointer named
    args = list(fake)
    args[2] = None
    assert L.w4a16_moe_forward(*args, ctypes.byref(d), ws, need, None) == 1
    assert b"w13_scales" in L.w4a16_last_error_message()
    # misaligned packed weights named
    args = list(fake)
    args[1] = P(0x10008)
    assert L.w4a16_moe_forward(*args, ctypes.byref(d), ws, need, None) == 1
    assert b"w13_packed" in L.w4a16_last_error_message()
    # workspace too small
    assert L.w4a16_moe_forward(*fake, ctypes.byref(d), ws, need - 1, None) == 3
    assert b"workspace" in L.w4a16_last_error_message()
    # zero tokens: nothing enqueued, OK even with null pointers
    d0 = good(num_tokens=0)
    assert L.w4a16_moe_forward(*([None] * 8), ctypes.byref(d0), None, 0, None) == 0


def test_prepare_routes_and_unpack_argument_errors():
    L = B.lib()
    d = good()
    P = ctypes.c_void_p
    args = [P(0x1000)] * 4
    assert L.w4a16_moe_prepare_routes(ctypes.byref(d), P(0x1000), 0, *args[:3], 100, args[3],
                                      None, None) == 1
    assert b"block_m" in L.w4a16_last_error_message()
    assert L.w4a16_moe_prepare_routes(ctypes.byref(d), P(0x1000), 16, *args[:3], 10, args[3],
                                      None, None) == 1
    assert b"capacity" in L.w4a16_last_error_message()
    assert L.w4a16_unpack_int4(None, 16, P(0x1000), None) == 1
    assert L.w4a16_unpack_int4(P(0x1000), -1, P(0x1000), None) == 1
    assert L.w4a16_unpack_int4(None, 0, None, None) == 0
    # FP4 decode: size, dtype and pointers checked before any launch
    assert L.w4a16_decode_fp4(P(0x1000), -1, 0, P(0x1000), None) == 1
    assert L.w4a16_decode_fp4(P(0x1000), 16, 7, P(0x1000), None) == 1
    assert b"dtype" in L.w4a16_last_error_message()
    assert L.w4a16_decode_fp4(None, 16, 0, P(0x1000), None) == 1
    assert L.w4a16_decode_fp4(P(0x1000), 16, 1, None, None) == 1
    assert L.w4a16_decode_fp4(None, 0, 0, None, None) == 0


def test_plans_by_route_count():
    # decode: small-batch path, the reduction split over 8 waves in 128-blocks
    p1 = B.get_plan(B.make_desc(num_tokens=1, hidden=7168, intermediate=256,
                                num_local_experts=384, top_k=8))
    assert p1.path == 2 and p1.k_slice == 7 * 128
    # prefill: grouped path with 64-row expert tiles
    p2 = B.get_plan(B.make_desc(num_tokens=2048, hidden=7168, intermediate=256,
                                num_local_experts=384, top_k=8))
    assert p2.path == 1 and p2.block_m == 64
    assert p2.max_positions == 2048 * 8 + 384 * 63
    assert p2.splitk_chunks == 0          # ~43 routes per expert: streaming gate/up
    # few routes per expert: split-K gate/up; chunks of an even number of
    # blocks, at most 18 (the x slice stays in LDS): 56 blocks -> 4 x 14
    p4 = B.get_plan(B.make_desc(num_tokens=32, hidden=7168, intermediate=256,
                                num_local_experts=384, top_k=8))
    assert p4.path == 1 and p4.splitk_chunks == 4
    assert B.get_plan(B.make_desc(num_tokens=256, hidden=7168, intermediate=256,
                                  num_local_experts=384, top_k=8)).splitk_chunks == 0
    d5 = B.make_desc(num_tokens=32, hidden=7168, intermediate=256, num_local_experts=384,
                     top_k=8, force_splitk=2)
    assert B.get_plan(d5).splitk_chunks == 0
    assert B.workspace_size(d5) < B.workspace_size(B.make_desc(
        num_tokens=32, hidden=7168, intermediate=256, num_local_experts=384, top_k=8))
    # forcing is honoured and the workspace follows the plan
    d = B.make_desc(num_tokens=16, hidden=256, intermediate=384, num_local_experts=8, top_k=2,
                    force_block_m=64, force_path=1)
    p3 = B.get_plan(d)
    assert (p3.path, p3.block_m) == (1, 64)
    assert p3.workspace_bytes == B.workspace_size(d)


def test_fp16_route_choice():
    """The fp16 route is opt-in (descriptor field fp16_route = 1); the default
    plan forms every product with per-group scaling.  Opted in, the grouped
    path's streaming launches take it when the expected valid routes per
    touched expert, R / (E (1 - (1 - 1/E)^R)) with R = T K scaled by the local
    share, reach 16; only for bf16 activations with group scales.  Its rerun
    flags sit in the workspace."""
    kimi = dict(hidden=7168, intermediate=256, num_local_experts=384, top_k=8)
    for T in (1, 32, 256, 1024, 2048):
        pl = B.get_plan(B.make_desc(num_tokens=T, **kimi))
        assert (pl.fp16_route, pl.rerun_flags_up, pl.rerun_flags_down,
                pl.rerun_flags_offset) == (0, 0, 0, 0), T
    for T, want in ((1, 0), (32, 0), (256, 0), (512, 0), (1024, 3), (2048, 3)):
        # 512 tokens: 10.7 routes per touched expert; 1024: 21.3
        pl = B.get_plan(B.make_desc(num_tokens=T, fp16_route=1, **kimi))
        assert pl.fp16_route == want, (T, pl.fp16_route)
        if want:
            assert pl.rerun_flags_up > 0 and pl.rerun_flags_down > 0
            assert 0 < pl.rerun_flags_offset
            assert (pl.rerun_flags_offset + 4 * max(pl.rerun_flags_up, pl.rerun_flags_down)
                    <= pl.workspace_bytes)
        else:
            assert (pl.rerun_flags_up, pl.rerun_flags_down, pl.rerun_flags_offset) == (0, 0, 0)
    assert B.get_plan(B.make_desc(num_tokens=2048, dtype=torch.float16, fp16_route=1,
                                  **kimi)).fp16_route == 0
    assert B.get_plan(B.make_desc(num_tokens=2048, per_channel=True, fp16_route=1,
                                  **kimi)).fp16_route == 0
    # a local share of 32 of 256 experts: 512 tokens give 4096 routes, 512
    # of them valid in expectation, 16 per local expert
    share = dict(hidden=7168, intermediate=2048, num_local_experts=32, top_k=8,
                 num_global_experts=256, fp16_route=1)
    assert B.get_plan(B.make_desc(num_tokens=256, **share)).fp16_route == 0
    assert B.get_plan(B.make_desc(num_tokens=512, **share)).fp16_route == 3
    # counted as if every route were local, 256 tokens would already qualify
    assert B.get_plan(B.make_desc(num_tokens=256, **dict(share, num_global_experts=0))).fp16_route == 3


def test_buffer_offset_limits():
    # x at 2^31 bytes or more: 32-bit buffer offsets cannot address it
    d = B.make_desc(num_tokens=65536 // 2, hidden=32768, intermediate=256,
                    num_local_experts=8, top_k=1)
    with pytest.raises(B.W4A16Error) as ei:
        B.workspace_size(d)
    assert ei.value.status == 2 and "x:" in str(ei.value)
    # one token fewer fits
    d.num_tokens = 65536 // 2 - 1
    assert B.workspace_size(d) > 0


def test_small_batch_path_only_for_short_intermediate():
    kimi = dict(hidden=7168, intermediate=256, num_local_experts=384, top_k=8)
    assert B.get_plan(B.make_desc(num_tokens=1, **kimi)).path == 2
    assert B.get_plan(B.make_desc(num_tokens=8, **kimi)).path == 2
    # I = 2048, top-8, every route local: the grouped path even for 1 token,
    # with the streaming gate/up (16 column tiles per expert tile; forced
    # split-K measured 107 us against 81)
    ds = dict(hidden=7168, intermediate=2048, num_local_experts=32, top_k=8)
    p = B.get_plan(B.make_desc(num_tokens=1, **ds))
    assert p.path == 1 and p.splitk_chunks == 0
    # the same experts as a share of 256 global ones (one local route per
    # token expected): the small-batch path up to 96 routes (past them most
    # of its gate/up workgroups would own no local expert)
    for T in (1, 8, 12):
        assert B.get_plan(B.make_desc(num_tokens=T, num_global_experts=256, **ds)).path == 2
    assert B.get_plan(B.make_desc(num_tokens=13, num_global_experts=256, **ds)).path == 1
    # every route local: the small-batch path up to 128 routes
    for T in (9, 16):
        assert B.get_plan(B.make_desc(num_tokens=T, **kimi)).path == 2
    assert B.get_plan(B.make_desc(num_tokens=17, **kimi)).path == 1
    # a quarter local: 2 expected local routes x I = 4096, small batch; two
    # thirds local: 5.3 x I = 10,923, still small batch; four fifths local:
    # 6.4 x I = 13,107 > 12,288, grouped
    assert B.get_plan(B.make_desc(num_tokens=1, num_global_experts=128, **ds)).path == 2
    assert B.get_plan(B.make_desc(num_tokens=1, num_global_experts=48, **ds)).path == 2
    assert B.get_plan(B.make_desc(num_tokens=1, num_global_experts=40, **ds)).path == 1


def test_small_batch_path_bounded_by_its_working_workgroups():
    """Past a few tokens the small-batch gate/up grid's working workgroups,
    (N1 / 16) x the local experts expected, decide: at most 7,400."""
    pc = S.WORKLOADS["per_channel"]     # N1 / 16 = 176, 60 experts
    assert B.get_plan(B.desc_for(pc, 16)).path == 2    # about 6,970
    assert B.get_plan(B.desc_for(pc, 24)).path == 1    # about 8,450
    r2 = S.WORKLOADS["relu2_skew"]      # N1 / 16 = 116, 128 experts, top-6, I = 1856
    for T in (1, 8):
        assert B.get_plan(B.desc_for(r2, T)).path == 2
    assert B.get_plan(B.desc_for(r2, 16)).path == 1    # about 7,790


def test_small_batch_path_limits():
    # more than 128 routes (two ballots of one wave) cannot take the
    # small-batch path
    d = B.make_desc(num_tokens=17, hidden=256, intermediate=384, num_local_experts=8, top_k=8,
                    force_path=2)
    with pytest.raises(B.W4A16Error) as ei:
        B.workspace_size(d)
    assert ei.value.status == 2 and "routes" in ei.value.message
    d.num_tokens = 16
    assert B.get_plan(d).path == 2
    # hidden sizes beyond 8 waves x 1024 cannot take it either
    d2 = B.make_desc(num_tokens=1, hidden=8256, intermediate=384, num_local_experts=8, top_k=2,
                     force_path=2)
    with pytest.raises(B.W4A16Error) as ei:
        B.workspace_size(d2)
    assert "hidden" in ei.value.message
    d2.force_path = 0
    assert B.get_plan(d2).path == 1


def test_fp16_route_exact_scale_range():
    """The fp16 route forms q * s as (24 + q)/16 * 16s - 24s with one rounding
    to fp16, exact when 16s, 24s and every q * s (q in [-8, 7]) are fp16
    values.  Over every finite bf16 magnitude that holds exactly on
    [2^-17, 2720] (bf16 bits 0x3700 to 0x452A), the range the kernels accept,
    and fails just outside it."""
    import numpy as np
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    s = (bits << 16).view(np.float32).astype(np.float64)

    def rep(v):  # v exactly an fp16 value (finite)
        with np.errstate(over="ignore"):
            h = v.astype(np.float16)
        return np.isfinite(h) & (h.astype(np.float64) == v)

    ok = rep(16.0 * s) & rep(24.0 * s)
    for q in range(-8, 8):
        ok &= rep(q * s)
    lo, end = 0x3700, 0x452B
    inside = (bits >= lo) & (bits < end)
    assert ok[inside].all()
    assert not ok[bits == end].any() and not ok[bits == lo - 1].any()
    assert not ok[bits >= end].any()


def test_forward_rejects_wrong_out_shape(monkeypatch):
    """An `out` of the wrong shape is refused by the binding before the
    library is called (the kernels write T * H values through its pointer).
    The device checks are bypassed so the shape check runs on host tensors;
    the library would be reached only past it."""
    import numpy as np  # noqa: F401
    monkeypatch.setattr(B, "_dev", lambda *a, **k: None)
    called = []
    monkeypatch.setattr(B, "_check", lambda st: called.append(st))
    T, H, I, E, K = 4, 256, 384, 8, 2
    x = torch.zeros(T, H, dtype=torch.bfloat16)
    w13 = torch.zeros(E, 2 * I, H // 2, dtype=torch.uint8)
    s13 = torch.zeros(E, 2 * I, H // 32, dtype=torch.bfloat16)
    w2 = torch.zeros(E, H, I // 2, dtype=torch.uint8)
    s2 = torch.zeros(E, H, I // 32, dtype=torch.bfloat16)
    ids = torch.zeros(T, K, dtype=torch.int32)
    wts = torch.zeros(T, K, dtype=torch.float32)
    for bad in ((T - 1, H), (T, H - 8), (T * H,)):
        with pytest.raises(ValueError, match="out: shape"):
            B.moe_forward(x, w13, s13, w2, s2, ids, wts, intermediate=I, num_local_experts=E,
                          out=torch.zeros(*bad, dtype=torch.bfloat16))
    # only the host-side workspace query ran, never the forward
    assert all(st == 0 for st in called)


def test_no_alloc_forward_rejects_before_anything():
    """The no-alloc forward checks the descriptor and the scratch limit before
    it touches a pointer or the device (so this runs without a GPU)."""
    L = B.lib()
    small = B.make_desc(num_tokens=4, hidden=256, intermediate=384, num_local_experts=8, top_k=2)
    big = B.make_desc(num_tokens=2048, hidden=7168, intermediate=256, num_local_experts=384,
                      top_k=8)
    assert B.workspace_size(small) <= B.NOALLOC_SCRATCH_BYTES < B.workspace_size(big)
    st = L.w4a16_moe_forward_noalloc(*([None] * 8), ctypes.byref(big), None)
    assert st == 2 and "no-alloc scratch" in L.w4a16_last_error_message().decode()
    bad = B.make_desc(num_tokens=-1, hidden=256, intermediate=384, num_local_experts=8, top_k=2)
    assert L.w4a16_moe_forward_noalloc(*([None] * 8), ctypes.byref(bad), None) == 1


def test_routed_forward_argument_errors():
    """The routed forward and route_and_prepare check the router arguments on
    the host before anything is enqueued (no GPU needed)."""
    L = B.lib()
    P = ctypes.c_void_p
    d = B.make_desc(num_tokens=4, hidden=256, intermediate=384, num_local_experts=8, top_k=2,
                    num_global_experts=2000)
    args = [P(0x1000)] * 5 + [P(0x1000), 0, P(0x1000), P(0x1000), P(0x1000), ctypes.byref(d),
                              P(0x1000), 1 << 30, None, None, 0]
    assert L.w4a16_moe_forward_routed(*args) == 2
    assert "num_global_experts=2000" in L.w4a16_last_error_message().decode()
    d.num_global_experts = 8
    args[6] = 2
    assert L.w4a16_moe_forward_routed(*args) == 1
    assert "renormalize" in L.w4a16_last_error_message().decode()
    args[6] = 0
    args[5] = None
    assert L.w4a16_moe_forward_routed(*args) == 1
    assert "router_logits" in L.w4a16_last_error_message().decode()
    d.top_k = 9           # more than the 8 global experts
    st = L.w4a16_moe_route_and_prepare(ctypes.byref(d), P(0x1000), 0, 64, P(0x1000), P(0x1000),
                                       P(0x1000), P(0x1000), P(0x1000), 1 << 20, P(0x1000), None,
                                       None)
    assert st == 2 and "top_k=9" in L.w4a16_last_error_message().decode()


def test_fp4_layout_descriptor():
    """The FP4 group layout is accepted with group 32 and takes the INT4 group
    layout's workspace; it never takes the fp16 route."""
    kimi = dict(hidden=7168, intermediate=256, num_local_experts=384, top_k=8)
    for T in (1, 32, 2048):
        a = B.make_desc(num_tokens=T, **kimi)
        f = B.make_desc(num_tokens=T, fp4=True, **kimi)
        assert f.qlayout == 2
        assert B.workspace_size(f) == B.workspace_size(a)
        assert B.get_plan(f).path == B.get_plan(a).path
    assert B.get_plan(B.make_desc(num_tokens=2048, fp4=True, fp16_route=1, **kimi)).fp16_route == 0
    bad = B.make_desc(num_tokens=4, hidden=256, intermediate=384, num_local_experts=8, top_k=2,
                      fp4=True, group_size=16)
    with pytest.raises(B.W4A16Error) as ei:
        B.workspace_size(bad)
    assert ei.value.status == 2 and "group_size" in ei.value.message


def test_repack_per_channel_argument_errors():
    L = B.lib()
    P = ctypes.c_void_p
    p = P(0x1000)
    assert L.w4a16_repack_per_channel(p, p, 2, 63, 128, p, p, None) == 1
    assert b"n_out" in L.w4a16_last_error_message()
    assert L.w4a16_repack_per_channel(p, p, 2, 64, 96, p, p, None) == 2
    assert b"k_in" in L.w4a16_last_error_message()
    assert L.w4a16_repack_per_channel(p, None, 2, 64, 128, p, p, None) == 1
    assert b"scales" in L.w4a16_last_error_message()
    assert L.w4a16_repack_per_channel(p, p, 2, 64, 128, P(0x1002), p, None) == 1
    assert b"aligned" in L.w4a16_last_error_message()
    assert L.w4a16_repack_per_channel(p, p, -1, 64, 128, p, p, None) == 1
    # no experts: nothing enqueued, OK with null pointers
    assert L.w4a16_repack_per_channel(None, None, 0, 64, 128, None, None, None) == 0


def test_tile_order_chosen_between_9_and_80_routes_per_expert():
    """The grouped path takes tiles biggest first where tile sizes mix and the
    launch has more than one round of workgroups (one per CU)."""
    wl = S.WORKLOADS["kimi_tp8"]
    for T, want in ((256, 0), (512, 1), (1024, 1), (2048, 1), (4096, 0)):
        assert B.get_plan(B.desc_for(wl, T)).tile_order == want, T
    assert B.get_plan(B.desc_for(wl, 8)).tile_order == 0   # small batch
    r2 = S.WORKLOADS["relu2_skew"]
    assert B.get_plan(B.desc_for(r2, 1024)).tile_order == 1   # 48 routes per expert
    assert B.get_plan(B.desc_for(r2, 2048)).tile_order == 0   # 96: mostly full tiles
    assert B.get_plan(B.desc_for(r2, 4096)).tile_order == 0
    # 64 routes per expert, but 24 workgroups: one round, no tail to shorten
    assert B.get_plan(B.desc_for(S.WORKLOADS["tiny"], 256)).tile_order == 0


def test_activations_formed_in_the_down_launch_after_split_k():
    """Split-K gate/up followed by the resident down kernel runs no activation
    launch; the streaming gate/up, or a down GEMM that does not hold the
    reduction in LDS, keeps it."""
    wl = S.WORKLOADS["kimi_tp8"]
    for T, want in ((32, 1), (64, 1), (48, 0), (128, 0), (256, 0), (2048, 0)):
        p = B.get_plan(B.desc_for(wl, T))
        assert p.act_in_down == want, T
        assert want == 0 or p.splitk_chunks > 0
    assert B.get_plan(B.desc_for(wl, 8)).act_in_down == 0   # small batch
    # forced split-K at 256 tokens still pairs with the resident down kernel
    assert B.get_plan(B.desc_for(wl, 256, force_path=1, force_splitk=1)).act_in_down == 1
    for name, wl in S.WORKLOADS.items():
        for T in (32, 256):
            p = B.get_plan(B.desc_for(wl, T))
            if p.act_in_down:
                assert p.splitk_chunks > 0 and wl.inter <= 256, (name, T)


def test_split_k_only_where_the_streaming_grid_underfills():
    """Split-K gate/up is chosen for few routes per expert, a resident down
    kernel, and a streaming grid (touched experts x column tiles, one
    workgroup per CU) whose last round would be less than 0.8 full."""
    wl = S.WORKLOADS["kimi_tp8"]
    # 2 column tiles per expert tile; expected touched experts of 384
    for T, want in ((32, True), (48, False), (64, True), (80, False), (96, False), (128, False)):
        p = B.get_plan(B.desc_for(wl, T))
        assert (p.splitk_chunks > 0) == want, T
    # larger intermediates: the streaming kernel at every token count
    for name in ("deepseek_local", "relu2_skew", "per_channel"):
        for T in (16, 32, 48, 64, 96, 128):
            p = B.get_plan(B.desc_for(S.WORKLOADS[name], T))
            assert p.splitk_chunks == 0, (name, T)
    # forcing still selects either form
    assert B.get_plan(B.desc_for(wl, 128, force_path=1, force_splitk=1)).splitk_chunks > 0
    assert B.get_plan(B.desc_for(wl, 32, force_path=1, force_splitk=2)).splitk_chunks == 0
