"""CPU oracle for the local W4A16 mixture-of-experts forward (test infrastructure).

TEST INFRASTRUCTURE ONLY: this package may be imported by ``tests/``, by the
smoke check in ``__graft_entry__.py`` and by the CPU-baseline leg of
``bench.py``.  The product path (the HIP library and its Python binding) never
imports it.

The arithmetic lives in ``moe_oracle.c`` (plain C, FP32, built with
``-ffp-contract=off``); this module only marshals numpy arrays through ctypes.
16-bit floating-point arrays (bf16 or fp16) travel as their raw ``uint16`` bit
patterns, selected by ``dtype`` (0 = bf16, 1 = fp16).

Parity pins for every function are in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DT_BF16, DT_FP16 = 0, 1
ACT_SILU_GATED, ACT_RELU2 = 0, 1
Q_GROUP_K, Q_PER_CHANNEL, Q_FP4_GROUP_K = 0, 1, 2


def build() -> str:
    """Compile the oracle with gcc (idempotent; called by the build step)."""
    subprocess.run(["make", "-s", "-C", _HERE, "liboracle.so"], check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(
        os.path.join(_HERE, "moe_oracle.c")
    ):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.oracle_h16_to_f32.argtypes = [P, i64, i32, P]
    lib.oracle_f32_to_h16.argtypes = [P, i64, i32, P]
    lib.oracle_unpack_int4.argtypes = [P, i64, P]
    lib.oracle_pack_int4.argtypes = [P, i64, P]
    lib.oracle_quantize_group.argtypes = [P, i64, i64, i32, i32, P, P]
    lib.oracle_quantize_per_channel.argtypes = [P, i64, i64, i32, P, P]
    lib.oracle_dequant_matrix.argtypes = [P, P, i64, i64, i32, i32, i32, P]
    lib.oracle_prepare_routes.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, i64, P]
    lib.oracle_prepare_routes.restype = i64
    lib.oracle_moe_forward.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                       P, P, P, P, P, P, P, P, P, i32]
    lib.oracle_moe_forward.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_route_topk.argtypes = [P, i64, i32, i32, i32, P, P]
    lib.oracle_unpack_fp4.argtypes = [P, i64, P]
    lib.oracle_repack_per_channel.argtypes = [P, P, i64, i64, P, P]
    lib.oracle_e8m0_to_f32.argtypes = [P, i64, P]
    lib.oracle_quantize_mxfp4.argtypes = [P, i64, i64, P, P]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def h16_to_f32(bits, dtype: int) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float32)
    _load().oracle_h16_to_f32(_p(bits), bits.size, dtype, _p(out))
    return out


def f32_to_h16(x, dtype: int) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_f32_to_h16(_p(x), x.size, dtype, _p(out))
    return out


def unpack_int4(packed) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] int8, low nibble first, two's complement."""
    packed = _c(packed, np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.int8)
    _load().oracle_unpack_int4(_p(packed), packed.size, _p(out))
    return out


def pack_int4(q) -> np.ndarray:
    """[..., 2n] int8 in [-8, 7] -> [..., n] bytes."""
    q = _c(q, np.int8)
    assert q.shape[-1] % 2 == 0
    out = np.empty(q.shape[:-1] + (q.shape[-1] // 2,), np.uint8)
    _load().oracle_pack_int4(_p(q), q.size, _p(out))
    return out


def quantize_group(w, group: int, dtype: int):
    """w [rows, cols] fp32 -> (q int8 [rows, cols], scale bits uint16 [rows, cols/group])."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows, cols // group), np.uint16)
    _load().oracle_quantize_group(_p(w), rows, cols, group, dtype, _p(q), _p(s))
    return q, s


def quantize_per_channel(w, dtype: int):
    """w [rows, cols] fp32 -> (q int8 [rows, cols], scale bits uint16 [rows])."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty((rows,), np.uint16)
    _load().oracle_quantize_per_channel(_p(w), rows, cols, dtype, _p(q), _p(s))
    return q, s


def dequant_matrix(packed, scales, n_out: int, k_in: int, layout: int, group: int,
                   dtype: int) -> np.ndarray:
    """One expert's packed matrix -> fp32 [n_out, k_in]."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    out = np.empty((n_out, k_in), np.float32)
    _load().oracle_dequant_matrix(_p(packed), _p(scales), n_out, k_in, layout, group, dtype,
                                  _p(out))
    return out


def prepare_routes(ids, num_experts: int, expert_offset: int, block_m: int):
    """Route tables: (counts [E], offsets [E+1], sorted [P], slot [T*K])."""
    ids = _c(ids, np.int32)
    T, K = ids.shape
    R = T * K
    cap = R + num_experts * (block_m - 1) + 1
    counts = np.empty(num_experts, np.int32)
    offsets = np.empty(num_experts + 1, np.int32)
    sorted_ = np.empty(max(cap, 1), np.int32)
    slot = np.empty(max(R, 1), np.int32)
    total = _load().oracle_prepare_routes(_p(ids), T, K, num_experts, expert_offset, block_m,
                                          _p(counts), _p(offsets), _p(sorted_), cap, _p(slot))
    assert total >= 0
    return counts, offsets, sorted_[:total].copy(), slot[:R].copy()


def moe_forward(x_bits, w13p, w13s, w2p, w2s, ids, wts, *, hidden: int, inter: int,
                num_experts: int, expert_offset: int = 0, group: int = 32,
                act: int = ACT_SILU_GATED, layout: int = Q_GROUP_K, dtype: int = DT_BF16,
                want_routes: bool = False, nthreads: int = 0):
    """FP32 MoE output [T, H] (and optionally the per-route outputs [T*K, H])."""
    x_bits = _c(x_bits, np.uint16)
    w13p, w2p = _c(w13p, np.uint8), _c(w2p, np.uint8)
    w13s, w2s = _c(w13s, np.uint16), _c(w2s, np.uint16)
    ids, wts = _c(ids, np.int32), _c(wts, np.float32)
    T, K = ids.shape
    assert x_bits.shape == (T, hidden)
    out = np.empty((T, hidden), np.float32)
    yr = np.full((max(T * K, 1), hidden), np.nan, np.float32) if want_routes else None
    rc = _load().oracle_moe_forward(T, hidden, inter, num_experts, expert_offset, K, group, act,
                                    layout, dtype, _p(x_bits), _p(w13p), _p(w13s), _p(w2p),
                                    _p(w2s), _p(ids), _p(wts), _p(out),
                                    _p(yr) if yr is not None else None, nthreads)
    assert rc == 0, "oracle allocation failed"
    return (out, yr[: T * K]) if want_routes else out


def route_topk(logits, top_k: int, renormalize: bool = False):
    """Router scoring: (ids int32 [T, K], weights fp32 [T, K]) from fp32
    logits [T, E_global]: softmax over all experts, the K largest in
    descending order (ties to the lower id), renormalized over the K if asked."""
    logits = _c(logits, np.float32)
    T, Eg = logits.shape
    ids = np.empty((T, top_k), np.int32)
    wts = np.empty((T, top_k), np.float32)
    _load().oracle_route_topk(_p(logits), T, Eg, top_k, 1 if renormalize else 0, _p(ids),
                              _p(wts))
    return ids, wts


def unpack_fp4(packed) -> np.ndarray:
    """E2M1 codes, two per byte (even index in the low nibble), as float32."""
    b = _c(packed, np.uint8).ravel()
    out = np.empty(2 * b.size, np.float32)
    _load().oracle_unpack_fp4(_p(b), b.size, _p(out))
    return out


def e8m0_to_f32(codes) -> np.ndarray:
    c = _c(codes, np.uint8).ravel()
    out = np.empty(c.size, np.float32)
    _load().oracle_e8m0_to_f32(_p(c), c.size, _p(out))
    return out.reshape(np.shape(codes))


def quantize_mxfp4(w):
    """MXFP4 along the last axis in blocks of 32: (packed uint8 [.., cols/2],
    E8M0 uint8 [.., cols/32])."""
    w = _c(w, np.float32)
    rows, cols = int(np.prod(w.shape[:-1])), w.shape[-1]
    packed = np.empty((rows, cols // 2), np.uint8)
    sc = np.empty((rows, cols // 32), np.uint8)
    _load().oracle_quantize_mxfp4(_p(w), rows, cols, _p(packed), _p(sc))
    return packed.reshape(*w.shape[:-1], cols // 2), sc.reshape(*w.shape[:-1], cols // 32)


def repack_per_channel(packed, scales):
    """Per-channel INT4 [E, n_out/2, k_in] + scales [E, n_out] -> group layout
    [E, n_out, k_in/2] + scales [E, n_out, k_in/32] (16-bit patterns)."""
    packed, scales = _c(packed, np.uint8), _c(scales, np.uint16)
    E, half, k_in = packed.shape
    n_out = 2 * half
    op = np.empty((E, n_out, k_in // 2), np.uint8)
    osc = np.empty((E, n_out, k_in // 32), np.uint16)
    for e in range(E):
        pe, se = np.ascontiguousarray(packed[e]), np.ascontiguousarray(scales[e])
        ope, ose = np.empty((n_out, k_in // 2), np.uint8), np.empty((n_out, k_in // 32), np.uint16)
        _load().oracle_repack_per_channel(_p(pe), _p(se), n_out, k_in, _p(ope), _p(ose))
        op[e], osc[e] = ope, ose
    return op, osc
