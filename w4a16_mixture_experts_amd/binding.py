"""Thin Python binding of the C ABI in include/w4a16_moe.h (ctypes).

Argument marshalling only: tensors are checked for device, dtype and
contiguity, then their data pointers and the current HIP stream are passed to
libw4a16moe.so.  Every step of the forward pass runs in the library's HIP
kernels; there is no fallback: if the library is missing, loading fails.
PyTorch provides device memory (outputs, workspace) and the stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16moe.so")

DT_BF16, DT_FP16 = 0, 1
ACT_SILU_GATED, ACT_RELU2 = 0, 1
Q_GROUP_K, Q_PER_CHANNEL, Q_FP4_GROUP_K = 0, 1, 2
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP"}
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024   # W4A16_NOALLOC_SCRATCH_BYTES


class MoeDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_tokens", "hidden", "intermediate", "num_local_experts", "expert_offset", "top_k",
        "group_size", "dtype", "act", "qlayout", "force_path", "force_block_m", "force_splitk",
        "num_global_experts", "fp16_route", "fused_finalize", "force_tile_order")]


class MoePlan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("k_slice", ctypes.c_int32), ("splitk_chunks", ctypes.c_int32),
                ("max_positions", ctypes.c_int64), ("max_tiles", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("fp16_route", ctypes.c_int32),
                ("rerun_flags_up", ctypes.c_int32), ("rerun_flags_down", ctypes.c_int32),
                ("fused_combine", ctypes.c_int32), ("rerun_flags_offset", ctypes.c_size_t),
                ("tile_order", ctypes.c_int32), ("act_in_down", ctypes.c_int32)]


class W4A16Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None


def lib():
    """Load libw4a16moe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m w4a16_mixture_experts_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pdesc = ctypes.POINTER(MoeDesc)
    L.w4a16_moe_workspace_size.argtypes = [pdesc, ctypes.POINTER(sz)]
    L.w4a16_moe_get_plan.argtypes = [pdesc, ctypes.POINTER(MoePlan)]
    L.w4a16_moe_forward.argtypes = [P, P, P, P, P, P, P, P, pdesc, P, sz, P]
    L.w4a16_moe_forward_timed.argtypes = [P, P, P, P, P, P, P, P, pdesc, P, sz, P, P, i32]
    L.w4a16_moe_prepare_routes.argtypes = [pdesc, P, i32, P, P, P, i64, P, P, P]
    L.w4a16_unpack_int4.argtypes = [P, i64, P, P]
    L.w4a16_decode_fp4.argtypes = [P, i64, i32, P, P]
    L.w4a16_moe_route_topk.argtypes = [P, i64, i32, i32, i32, P, P, P]
    L.w4a16_stream_probe.argtypes = [P, i64, i32, P, P]
    L.w4a16_moe_forward_noalloc.argtypes = [P, P, P, P, P, P, P, P, pdesc, P]
    L.w4a16_moe_forward_routed.argtypes = [P, P, P, P, P, P, i32, P, P, P, pdesc, P, sz, P, P,
                                           i32]
    L.w4a16_moe_route_and_prepare.argtypes = [pdesc, P, i32, i32, P, P, P, P, P, i64, P, P, P]
    L.w4a16_e8m0_to_scales.argtypes = [P, i64, i32, P, P]
    L.w4a16_repack_per_channel.argtypes = [P, P, i64, i32, i32, P, P, P]
    L.w4a16_status_string.argtypes = [i32]
    L.w4a16_status_string.restype = ctypes.c_char_p
    L.w4a16_last_error_message.restype = ctypes.c_char_p
    for f in ("w4a16_moe_workspace_size", "w4a16_moe_get_plan", "w4a16_moe_forward",
              "w4a16_moe_forward_timed",
              "w4a16_moe_prepare_routes", "w4a16_unpack_int4", "w4a16_decode_fp4", "w4a16_moe_route_topk",
              "w4a16_stream_probe", "w4a16_moe_forward_noalloc", "w4a16_moe_forward_routed",
              "w4a16_moe_route_and_prepare", "w4a16_e8m0_to_scales",
              "w4a16_repack_per_channel"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise W4A16Error(status, lib().w4a16_last_error_message().decode())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(name: str, t: torch.Tensor, dtypes, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def make_desc(*, num_tokens: int, hidden: int, intermediate: int, num_local_experts: int,
              top_k: int, expert_offset: int = 0, dtype=torch.bfloat16, gated: bool = True,
              per_channel: bool = False, fp4: bool = False, group_size: int = 32,
              force_path: int = 0,
              force_block_m: int = 0, force_splitk: int = 0,
              num_global_experts: int = 0, fp16_route: int = 0,
              fused_finalize: int = 0, force_tile_order: int = 0) -> MoeDesc:
    """force_path: 0 auto, 1 grouped, 2 small batch; force_block_m: 0 or 64;
    force_splitk: 0 auto, 1 split-K gate/up, 2 streaming gate/up (64-row tiles);
    num_global_experts: experts the routes are drawn over (0 = num_local_experts),
    used only to choose the variant; fp16_route: 1 opts in to the fp16 route
    (bf16 only; rows of activations all below about 2^-14 keep fewer bits);
    fused_finalize: 1 runs the combine inside the down GEMM launch (grouped path);
    force_tile_order: grouped path, 0 auto, 1 tiles in route order, 2 biggest first."""
    return MoeDesc(num_tokens, hidden, intermediate, num_local_experts, expert_offset, top_k,
                   group_size, DT_FP16 if dtype == torch.float16 else DT_BF16,
                   ACT_SILU_GATED if gated else ACT_RELU2,
                   Q_PER_CHANNEL if per_channel else (Q_FP4_GROUP_K if fp4 else Q_GROUP_K),
                   force_path, force_block_m,
                   force_splitk, num_global_experts, fp16_route, fused_finalize,
                   force_tile_order)


def workspace_size(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().w4a16_moe_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def get_plan(desc: MoeDesc) -> MoePlan:
    pl = MoePlan()
    _check(lib().w4a16_moe_get_plan(ctypes.byref(desc), ctypes.byref(pl)))
    return pl


def desc_for(wl, T: int, **force) -> MoeDesc:
    """Descriptor of a synthetic workload (w4a16_mixture_experts_amd.synth)."""
    return make_desc(num_tokens=T, hidden=wl.hidden, intermediate=wl.inter,
                     num_local_experts=wl.num_experts, top_k=wl.top_k,
                     expert_offset=wl.expert_offset, dtype=wl.dtype, gated=wl.gated,
                     per_channel=wl.per_channel, fp4=wl.fp4,
                     num_global_experts=wl.num_global_experts, **force)


def moe_forward(x, w13_packed, w13_scales, w2_packed, w2_scales, topk_ids, topk_weights, *,
                intermediate: int, num_local_experts: int, expert_offset: int = 0,
                gated: bool = True, per_channel: bool = False, fp4: bool = False, out=None,
                workspace=None,
                force_path: int = 0, force_block_m: int = 0, force_splitk: int = 0,
                num_global_experts: int = 0, fp16_route: int = 0, fused_finalize: int = 0,
                force_tile_order: int = 0,
                stream=None, stage_events=None, no_alloc: bool = False) -> torch.Tensor:
    """Local W4A16 MoE forward: returns out [T, H] in x's dtype.

    no_alloc: call w4a16_moe_forward_noalloc (the library's own scratch array
    instead of a workspace; `out` should then be passed in as well, since
    allocating it here would defeat the purpose).

    stage_events: optional list of up to 8 torch.cuda.Event(enable_timing=True);
    events 2i and 2i+1 are recorded around stage i (0 route preparation,
    1 gate/up GEMM, 2 down GEMM, 3 combine) on the stream the kernels use.
    """
    half = (torch.bfloat16, torch.float16)
    _dev("x", x, half)
    dev = x.device
    T, H = x.shape
    _dev("w13_packed", w13_packed, (torch.uint8,), dev)
    _dev("w2_packed", w2_packed, (torch.uint8,), dev)
    _dev("w13_scales", w13_scales, (x.dtype,), dev)
    _dev("w2_scales", w2_scales, (x.dtype,), dev)
    _dev("topk_ids", topk_ids, (torch.int32,), dev)
    _dev("topk_weights", topk_weights, (torch.float32,), dev)
    if topk_ids.dim() != 2 or topk_ids.shape[0] != T or topk_weights.shape != topk_ids.shape:
        raise ValueError("topk_ids/topk_weights: expected [T, K] matching x")
    E = num_local_experts
    I = intermediate
    N1 = 2 * I if gated else I
    if per_channel:
        want = {"w13_packed": (E, N1 // 2, H), "w13_scales": (E, N1),
                "w2_packed": (E, H // 2, I), "w2_scales": (E, H)}
    else:
        want = {"w13_packed": (E, N1, H // 2), "w13_scales": (E, N1, H // 32),
                "w2_packed": (E, H, I // 2), "w2_scales": (E, H, I // 32)}
    for name, t in (("w13_packed", w13_packed), ("w13_scales", w13_scales),
                    ("w2_packed", w2_packed), ("w2_scales", w2_scales)):
        if tuple(t.shape) != want[name]:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want[name]}")
    desc = make_desc(num_tokens=T, hidden=H, intermediate=I, num_local_experts=E,
                     top_k=topk_ids.shape[1], expert_offset=expert_offset, dtype=x.dtype,
                     gated=gated, per_channel=per_channel, fp4=fp4, force_path=force_path,
                     force_block_m=force_block_m, force_splitk=force_splitk,
                     num_global_experts=num_global_experts, fp16_route=fp16_route,
                     fused_finalize=fused_finalize, force_tile_order=force_tile_order)
    nbytes = workspace_size(desc)
    if out is None:
        out = torch.empty(T, H, dtype=x.dtype, device=dev)
    else:
        _dev("out", out, (x.dtype,), dev)
        if tuple(out.shape) != (T, H):
            raise ValueError(f"out: shape {tuple(out.shape)}, expected {(T, H)}")
    if no_alloc:
        if workspace is not None or stage_events is not None:
            raise ValueError("no_alloc: takes no workspace and no stage events")
        _check(lib().w4a16_moe_forward_noalloc(
            _ptr(x), _ptr(w13_packed), _ptr(w13_scales), _ptr(w2_packed), _ptr(w2_scales),
            _ptr(topk_ids), _ptr(topk_weights), _ptr(out), ctypes.byref(desc), _stream(stream)))
        return out
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    else:
        _dev("workspace", workspace, (torch.uint8,), dev)
    args = (_ptr(x), _ptr(w13_packed), _ptr(w13_scales), _ptr(w2_packed), _ptr(w2_scales),
            _ptr(topk_ids), _ptr(topk_weights), _ptr(out), ctypes.byref(desc), _ptr(workspace),
            workspace.numel(), _stream(stream))
    if stage_events is None:
        _check(lib().w4a16_moe_forward(*args))
    else:
        st = stream if stream is not None else torch.cuda.current_stream()
        for ev in stage_events:
            if ev is not None and not ev.cuda_event:
                ev.record(st)                 # torch creates its events lazily
        handles = (ctypes.c_void_p * len(stage_events))(
            *[ev.cuda_event if ev is not None else None for ev in stage_events])
        _check(lib().w4a16_moe_forward_timed(*args, handles, len(stage_events)))
    return out


def forward_workload(wl, W, tok, **kw) -> torch.Tensor:
    """moe_forward on synth.Weights / synth.Tokens already on the GPU."""
    return moe_forward(tok.x, W.w13_packed, W.w13_scales, W.w2_packed, W.w2_scales,
                       tok.topk_ids, tok.topk_weights, intermediate=wl.inter,
                       num_local_experts=wl.num_experts, expert_offset=wl.expert_offset,
                       gated=wl.gated, per_channel=wl.per_channel, fp4=wl.fp4,
                       num_global_experts=wl.num_global_experts, **kw)


ROUTE_CHUNKS_MAX = 32


def prepare_routes(topk_ids: torch.Tensor, num_local_experts: int, expert_offset: int,
                   block_m: int, stream=None, chunked: bool = True):
    """Route tables from the device kernels: (counts, offsets, sorted, slot).
    chunked: rank in parallel chunks as the forward does (else one chunk)."""
    _dev("topk_ids", topk_ids, (torch.int32,))
    T, K = topk_ids.shape
    R = T * K
    E = num_local_experts
    dev = topk_ids.device
    cap = R + min(E, R) * (block_m - 1)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    srt = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    slot = torch.empty(max(R, 1), dtype=torch.int32, device=dev)
    desc = MoeDesc(T, 64, 64, E, expert_offset, K, 32, 0, 0, 0, 0, 0, 0)
    scratch = (torch.empty(ROUTE_CHUNKS_MAX * E, dtype=torch.int32, device=dev)
               if chunked else None)
    _check(lib().w4a16_moe_prepare_routes(ctypes.byref(desc), _ptr(topk_ids), block_m,
                                          _ptr(counts), _ptr(offsets), _ptr(srt), cap,
                                          _ptr(slot), _ptr(scratch) if chunked else None,
                                          _stream(stream)))
    return counts, offsets, srt, slot[:R]


def unpack_int4(packed: torch.Tensor, stream=None) -> torch.Tensor:
    _dev("packed", packed, (torch.uint8,))
    out = torch.empty(packed.numel() * 2, dtype=torch.int8, device=packed.device)
    _check(lib().w4a16_unpack_int4(_ptr(packed), packed.numel(), _ptr(out), _stream(stream)))
    return out


def decode_fp4(packed: torch.Tensor, dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    """E2M1 codes (two per byte, the even index in the low nibble) through the
    GEMMs' device conversion, as float32."""
    _dev("packed", packed, (torch.uint8,))
    out = torch.empty(packed.numel() * 2, dtype=torch.float32, device=packed.device)
    _check(lib().w4a16_decode_fp4(_ptr(packed), packed.numel(),
                                  DT_FP16 if dtype == torch.float16 else DT_BF16, _ptr(out),
                                  _stream(stream)))
    return out


def route_topk(logits: torch.Tensor, top_k: int, renormalize: bool = False, out=None,
               stream=None):
    """Router scoring: (topk_ids int32 [T, K], topk_weights fp32 [T, K]) from fp32
    logits [T, E_global] on the GPU (softmax over all experts, the K largest,
    ties to the lower id; renormalized over the K if asked)."""
    _dev("logits", logits, (torch.float32,))
    if logits.dim() != 2:
        raise ValueError("logits: expected [T, E_global]")
    T, Eg = logits.shape
    if out is None:
        ids = torch.empty(T, top_k, dtype=torch.int32, device=logits.device)
        wts = torch.empty(T, top_k, dtype=torch.float32, device=logits.device)
    else:
        ids, wts = out
        _dev("topk_ids", ids, (torch.int32,), logits.device)
        _dev("topk_weights", wts, (torch.float32,), logits.device)
        if tuple(ids.shape) != (T, top_k) or tuple(wts.shape) != (T, top_k):
            raise ValueError("out: expected two [T, top_k] tensors")
    _check(lib().w4a16_moe_route_topk(_ptr(logits), T, Eg, top_k, 1 if renormalize else 0,
                                      _ptr(ids), _ptr(wts), _stream(stream)))
    return ids, wts


def stream_probe(buf: torch.Tensor, nbytes: int, row_bytes: int, sink: torch.Tensor, stream=None):
    """Streaming-read probe over the first nbytes of buf (uint8, GPU)."""
    _dev("buf", buf, (torch.uint8,))
    _dev("sink", sink, (torch.int32,), buf.device)
    if nbytes > buf.numel():
        raise ValueError(f"nbytes: {nbytes} exceeds buf ({buf.numel()} bytes)")
    _check(lib().w4a16_stream_probe(_ptr(buf), nbytes, row_bytes, _ptr(sink), _stream(stream)))


def moe_forward_routed(x, w13_packed, w13_scales, w2_packed, w2_scales, router_logits, *,
                       top_k: int, intermediate: int, num_local_experts: int,
                       expert_offset: int = 0, gated: bool = True, per_channel: bool = False,
                       fp4: bool = False,
                       renormalize: bool = False, out=None, workspace=None, ids_out=None,
                       force_path: int = 0, force_splitk: int = 0, fp16_route: int = 0,
                       fused_finalize: int = 0, force_tile_order: int = 0, stream=None,
                       stage_events=None):
    """Forward with the router fused in: returns (out [T, H], topk_ids [T, K],
    topk_weights [T, K]); router_logits [T, E_global] fp32 (E_global is their
    width)."""
    half = (torch.bfloat16, torch.float16)
    _dev("x", x, half)
    dev = x.device
    T, H = x.shape
    _dev("router_logits", router_logits, (torch.float32,), dev)
    if router_logits.dim() != 2 or router_logits.shape[0] != T:
        raise ValueError("router_logits: expected [T, E_global] matching x")
    Eg = router_logits.shape[1]
    for name, t in (("w13_packed", w13_packed), ("w2_packed", w2_packed)):
        _dev(name, t, (torch.uint8,), dev)
    for name, t in (("w13_scales", w13_scales), ("w2_scales", w2_scales)):
        _dev(name, t, (x.dtype,), dev)
    E, I = num_local_experts, intermediate
    N1 = 2 * I if gated else I
    want = ({"w13_packed": (E, N1 // 2, H), "w13_scales": (E, N1), "w2_packed": (E, H // 2, I),
             "w2_scales": (E, H)} if per_channel else
            {"w13_packed": (E, N1, H // 2), "w13_scales": (E, N1, H // 32),
             "w2_packed": (E, H, I // 2), "w2_scales": (E, H, I // 32)})
    for name, t in (("w13_packed", w13_packed), ("w13_scales", w13_scales),
                    ("w2_packed", w2_packed), ("w2_scales", w2_scales)):
        if tuple(t.shape) != want[name]:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {want[name]}")
    desc = make_desc(num_tokens=T, hidden=H, intermediate=I, num_local_experts=E, top_k=top_k,
                     expert_offset=expert_offset, dtype=x.dtype, gated=gated,
                     per_channel=per_channel, fp4=fp4, force_path=force_path,
                     force_splitk=force_splitk,
                     num_global_experts=Eg, fp16_route=fp16_route, fused_finalize=fused_finalize,
                     force_tile_order=force_tile_order)
    nbytes = workspace_size(desc)
    if out is None:
        out = torch.empty(T, H, dtype=x.dtype, device=dev)
    else:
        _dev("out", out, (x.dtype,), dev)
        if tuple(out.shape) != (T, H):
            raise ValueError(f"out: shape {tuple(out.shape)}, expected {(T, H)}")
    if ids_out is None:
        ids = torch.empty(T, top_k, dtype=torch.int32, device=dev)
        wts = torch.empty(T, top_k, dtype=torch.float32, device=dev)
    else:
        ids, wts = ids_out
        _dev("topk_ids", ids, (torch.int32,), dev)
        _dev("topk_weights", wts, (torch.float32,), dev)
        if tuple(ids.shape) != (T, top_k) or tuple(wts.shape) != (T, top_k):
            raise ValueError("ids_out: expected two [T, top_k] tensors")
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    else:
        _dev("workspace", workspace, (torch.uint8,), dev)
    st = stream if stream is not None else torch.cuda.current_stream()
    handles, n_ev = None, 0
    if stage_events is not None:
        for ev in stage_events:
            if ev is not None and not ev.cuda_event:
                ev.record(st)
        handles = (ctypes.c_void_p * len(stage_events))(
            *[ev.cuda_event if ev is not None else None for ev in stage_events])
        n_ev = len(stage_events)
    _check(lib().w4a16_moe_forward_routed(
        _ptr(x), _ptr(w13_packed), _ptr(w13_scales), _ptr(w2_packed), _ptr(w2_scales),
        _ptr(router_logits), 1 if renormalize else 0, _ptr(ids), _ptr(wts), _ptr(out),
        ctypes.byref(desc), _ptr(workspace), workspace.numel(), _stream(st), handles, n_ev))
    return out, ids, wts


def forward_workload_routed(wl, W, tok, **kw):
    """moe_forward_routed on synth.Weights / synth.Tokens already on the GPU
    (the tokens' router logits instead of their ids and weights)."""
    return moe_forward_routed(tok.x, W.w13_packed, W.w13_scales, W.w2_packed, W.w2_scales,
                              tok.logits, top_k=wl.top_k, intermediate=wl.inter,
                              num_local_experts=wl.num_experts, expert_offset=wl.expert_offset,
                              gated=wl.gated, per_channel=wl.per_channel, fp4=wl.fp4, **kw)


def route_and_prepare(logits: torch.Tensor, top_k: int, num_local_experts: int,
                      expert_offset: int, block_m: int, renormalize: bool = False, stream=None,
                      chunked: bool = True):
    """Routing fused with route preparation: (ids, weights, counts, offsets,
    sorted, slot) from the device kernels."""
    _dev("logits", logits, (torch.float32,))
    T, Eg = logits.shape
    R = T * top_k
    E = num_local_experts
    dev = logits.device
    cap = R + min(E, R) * (block_m - 1)
    ids = torch.empty(T, top_k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, top_k, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    srt = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    slot = torch.empty(max(R, 1), dtype=torch.int32, device=dev)
    desc = make_desc(num_tokens=T, hidden=64, intermediate=64, num_local_experts=E, top_k=top_k,
                     expert_offset=expert_offset, num_global_experts=Eg)
    scratch = (torch.empty(ROUTE_CHUNKS_MAX * E, dtype=torch.int32, device=dev)
               if chunked else None)
    _check(lib().w4a16_moe_route_and_prepare(
        ctypes.byref(desc), _ptr(logits), 1 if renormalize else 0, block_m, _ptr(ids), _ptr(wts),
        _ptr(counts), _ptr(offsets), _ptr(srt), cap, _ptr(slot),
        _ptr(scratch) if chunked else None, _stream(stream)))
    return ids, wts, counts, offsets, srt, slot[:R]


def e8m0_to_scales(e8m0: torch.Tensor, dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    """MXFP4 block scales (E8M0 codes) -> 16-bit scales 2^(e - 127) on the GPU."""
    _dev("e8m0", e8m0, (torch.uint8,))
    out = torch.empty(e8m0.shape, dtype=dtype, device=e8m0.device)
    _check(lib().w4a16_e8m0_to_scales(_ptr(e8m0), e8m0.numel(),
                                      DT_FP16 if dtype == torch.float16 else DT_BF16, _ptr(out),
                                      _stream(stream)))
    return out


def repack_per_channel(packed: torch.Tensor, scales: torch.Tensor, stream=None):
    """Per-channel INT4 [E, N/2, K] + scales [E, N] -> the group layout
    [E, N, K/2] + scales [E, N, K/32] (setup-only, on the GPU)."""
    _dev("packed", packed, (torch.uint8,))
    _dev("scales", scales, (torch.bfloat16, torch.float16), packed.device)
    E, half, K = packed.shape
    N = 2 * half
    if tuple(scales.shape) != (E, N):
        raise ValueError(f"scales: shape {tuple(scales.shape)}, expected {(E, N)}")
    op = torch.empty(E, N, K // 2, dtype=torch.uint8, device=packed.device)
    osc = torch.empty(E, N, K // 32, dtype=scales.dtype, device=packed.device)
    _check(lib().w4a16_repack_per_channel(_ptr(packed), _ptr(scales), E, N, K, _ptr(op), _ptr(osc),
                                          _stream(stream)))
    return op, osc
