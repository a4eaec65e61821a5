"""Plain CPU oracle for the W4AFP8 fused-MoE forward (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product (the HIP library and
its Python binding) never imports it, and this package never imports the
product: the two share no code.  The arithmetic lives in ``w4a8_oracle.c``
(plain single-threaded C, fp64 accumulation); this module only compiles it
with gcc, loads it with ctypes and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a8_oracle.c")
_HDR = os.path.join(_HERE, "w4a8_oracle.h")
LIB_PATH = os.path.join(_HERE, "liborc_w4a8.so")
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared"]

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liborc_w4a8.so``."""
    if not force and os.path.exists(LIB_PATH) and \
            os.path.getmtime(LIB_PATH) >= max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _p(arr, ctype):
    return arr.ctypes.data_as(ctypes.POINTER(ctype)) if arr is not None else None


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            L = ctypes.CDLL(LIB_PATH)
            i64, u8p, u16p = ctypes.c_int64, ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_uint16)
            f32p, f64p, i32p = ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)
            L.orc_e4m3_decode.restype = ctypes.c_double
            L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.orc_e4m3_encode.restype = ctypes.c_uint8
            L.orc_e4m3_encode.argtypes = [ctypes.c_float]
            L.orc_int4_value.restype = ctypes.c_int
            L.orc_int4_value.argtypes = [ctypes.c_uint8, ctypes.c_int]
            L.orc_bf16_to_double.restype = ctypes.c_double
            L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
            L.orc_bf16_from_double.restype = ctypes.c_uint16
            L.orc_bf16_from_double.argtypes = [ctypes.c_double]
            L.orc_quantize_rows_bf16.restype = None
            L.orc_quantize_rows_bf16.argtypes = [u16p, i64, i64, i64, u8p, f32p]
            L.orc_quantize_rows_f32.restype = None
            L.orc_quantize_rows_f32.argtypes = [f32p, i64, i64, u8p, f32p]
            L.orc_moe_align.restype = ctypes.c_int
            L.orc_moe_align.argtypes = [i32p, i64, i64, i64, i64, i64, i32p, i32p, i32p, i32p,
                                        i32p, i32p, i32p]
            L.orc_gemm_f64.restype = None
            L.orc_gemm_f64.argtypes = [u8p, f32p, i64, i64, u8p, f32p, i64, f64p]
            L.orc_gemm_bf16.restype = None
            L.orc_gemm_bf16.argtypes = [u8p, f32p, i64, i64, u8p, f32p, i64, u16p]
            L.orc_fused_moe.restype = ctypes.c_int
            L.orc_fused_moe.argtypes = [u16p, i64, i64, i32p, f32p, i64, i64, i64, i64,
                                        u8p, f32p, u8p, f32p, u16p, u8p, f32p, f64p]
            L.orc_quantize_rows_bf16_static.restype = None
            L.orc_quantize_rows_bf16_static.argtypes = [u16p, i64, i64, i64, ctypes.c_float, u8p, f32p]
            L.orc_fused_moe_static.restype = ctypes.c_int
            L.orc_fused_moe_static.argtypes = [u16p, i64, i64, i32p, f32p, i64, i64, i64, i64,
                                               u8p, f32p, u8p, f32p, f32p, f32p, u16p, u8p, f32p, f64p]
            L.orc_quantize_block_n.restype = None
            L.orc_quantize_block_n.argtypes = [f32p, ctypes.c_int, u8p, f32p]
            L.orc_gemm_ag_f64.restype = None
            L.orc_gemm_ag_f64.argtypes = [u8p, f32p, i64, i64, i64, u8p, f32p, u8p, i64, f64p]
            L.orc_fused_moe_recipe.restype = ctypes.c_int
            L.orc_fused_moe_recipe.argtypes = [u16p, i64, i64, i32p, f32p, i64, i64, i64, i64,
                                               ctypes.c_int, u8p, ctypes.c_void_p, u8p, ctypes.c_void_p,
                                               ctypes.c_int, u16p, u8p, f32p, f64p]
            L.orc_e2m1_decode.restype = ctypes.c_double
            L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
            L.orc_ue8m0_decode.restype = ctypes.c_double
            L.orc_ue8m0_decode.argtypes = [ctypes.c_uint8]
            L.orc_gemm_fp4_f64.restype = None
            L.orc_gemm_fp4_f64.argtypes = [u8p, f32p, i64, i64, u8p, u8p, i64, f64p]
            L.orc_swiglu.restype = None
            L.orc_swiglu.argtypes = [f64p, f64p, i64, f32p]
            L.orc_fused_moe_fp4.restype = ctypes.c_int
            L.orc_fused_moe_fp4.argtypes = [u16p, i64, i64, i32p, f32p, i64, i64, i64, i64,
                                            u8p, u8p, u8p, u8p, u16p, u8p, f32p, f64p]
            _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- codecs -----------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([L.orc_e4m3_decode(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_encode(values) -> np.ndarray:
    L = lib()
    v = np.asarray(values, dtype=np.float32)
    return np.array([L.orc_e4m3_encode(float(x)) for x in v.ravel()], dtype=np.uint8).reshape(v.shape)


def int4_value(byte: int, odd: int) -> int:
    return lib().orc_int4_value(int(byte), int(odd))


def e2m1_decode(nibbles) -> np.ndarray:
    L = lib()
    c = np.asarray(nibbles, dtype=np.uint8)
    return np.array([L.orc_e2m1_decode(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def ue8m0_decode(exps) -> np.ndarray:
    L = lib()
    c = np.asarray(exps, dtype=np.uint8)
    return np.array([L.orc_ue8m0_decode(int(x)) for x in c.ravel()], dtype=np.float64).reshape(c.shape)


def bf16_from_double(values) -> np.ndarray:
    L = lib()
    v = np.asarray(values, dtype=np.float64)
    return np.array([L.orc_bf16_from_double(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def bf16_to_double(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([L.orc_bf16_to_double(int(x)) for x in b.ravel()], dtype=np.float64).reshape(b.shape)


# ---- steps ------------------------------------------------------------------

def quantize_bf16(x_bits: np.ndarray):
    """bf16 bit patterns [M, K] -> (codes u8 [M, K], scales f32 [M, K/128])."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    codes = np.empty((M, K), np.uint8)
    scales = np.empty((M, K // 128), np.float32)
    lib().orc_quantize_rows_bf16(_p(x, ctypes.c_uint16), M, K, K, _p(codes, ctypes.c_uint8),
                                 _p(scales, ctypes.c_float))
    return codes, scales


def quantize_bf16_static(x_bits: np.ndarray, s: float):
    """bf16 bit patterns [M, K] with a static per-tensor scale s -> (codes, scales)."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    codes = np.empty((M, K), np.uint8)
    scales = np.empty((M, K // 128), np.float32)
    lib().orc_quantize_rows_bf16_static(_p(x, ctypes.c_uint16), M, K, K, float(np.float32(s)),
                                        _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_float))
    return codes, scales


def fused_moe_static(hidden_bits, topk_ids, topk_weights, expert_begin, num_local_experts,
                     w13, s13, w2, s2, a1_scale=None, a2_scale=None):
    """The forward with static per-tensor activation scales (None = dynamic)."""
    x = _c(hidden_bits, np.uint16)
    ids = _c(topk_ids, np.int32)
    tw = _c(topk_weights, np.float32)
    w13, w2 = _c(w13, np.uint8), _c(w2, np.uint8)
    s13, s2 = _c(s13, np.float32), _c(s2, np.float32)
    T, H = x.shape
    k = ids.shape[1]
    I = w2.shape[2] * 2
    a1 = None if a1_scale is None else np.array([a1_scale], np.float32)
    a2 = None if a2_scale is None else np.array([a2_scale], np.float32)
    out = np.empty((T, H), np.uint16)
    rc = lib().orc_fused_moe_static(_p(x, ctypes.c_uint16), T, H, _p(ids, ctypes.c_int32),
                                    _p(tw, ctypes.c_float), k, expert_begin, num_local_experts, I,
                                    _p(w13, ctypes.c_uint8), _p(s13, ctypes.c_float),
                                    _p(w2, ctypes.c_uint8), _p(s2, ctypes.c_float),
                                    _p(a1, ctypes.c_float), _p(a2, ctypes.c_float),
                                    _p(out, ctypes.c_uint16), None, None, None)
    if rc:
        raise ValueError("orc_fused_moe_static failed: %d" % rc)
    return out


def quantize_block_n(x: np.ndarray):
    """One block of n fp32 values -> (codes u8 [n], scale f32)."""
    x = _c(x, np.float32).ravel()
    codes = np.empty(x.size, np.uint8)
    sc = np.empty(1, np.float32)
    lib().orc_quantize_block_n(_p(x, ctypes.c_float), x.size, _p(codes, ctypes.c_uint8),
                               _p(sc, ctypes.c_float))
    return codes, sc[0]


def gemm_ag_f64(a, sa, ag, w, sw=None, sb=None) -> np.ndarray:
    """codes [M, K] with activation scales sa [M, K/ag] x int4 (sw [N, K/128])
    or fp4 (sb [N, K/32]) weights -> fp64 [M, N]."""
    a, sa, w = _c(a, np.uint8), _c(sa, np.float32), _c(w, np.uint8)
    M, K = a.shape
    N = w.shape[0]
    assert sa.shape == (M, K // ag) and (sw is None) != (sb is None)
    swc = None if sw is None else _c(sw, np.float32)
    sbc = None if sb is None else _c(sb, np.uint8)
    y = np.empty((M, N), np.float64)
    lib().orc_gemm_ag_f64(_p(a, ctypes.c_uint8), _p(sa, ctypes.c_float), ag, M, K,
                          _p(w, ctypes.c_uint8), _p(swc, ctypes.c_float), _p(sbc, ctypes.c_uint8), N,
                          _p(y, ctypes.c_double))
    return y


def fused_moe_recipe(hidden_bits, topk_ids, topk_weights, expert_begin, num_local_experts,
                     w13, s13, w2, s2, down_act_group, fp4=False, intermediates=False):
    """The forward with the down GEMM's input quantised per down_act_group K
    (128, 64 or 32); int4 (fp32 scales) or fp4 (UE8M0) weights."""
    x = _c(hidden_bits, np.uint16)
    ids = _c(topk_ids, np.int32)
    tw = _c(topk_weights, np.float32)
    sdt = np.uint8 if fp4 else np.float32
    w13, w2, s13, s2 = _c(w13, np.uint8), _c(w2, np.uint8), _c(s13, sdt), _c(s2, sdt)
    T, H = x.shape
    k = ids.shape[1]
    E = num_local_experts
    I = w2.shape[2] * 2
    out = np.empty((T, H), np.uint16)
    P = T * k
    qh = sh = y2 = None
    if intermediates:
        qh = np.zeros((max(P, 1), I), np.uint8)
        sh = np.zeros((max(P, 1), I // down_act_group), np.float32)
        y2 = np.zeros((max(P, 1), H), np.float64)
    rc = lib().orc_fused_moe_recipe(_p(x, ctypes.c_uint16), T, H, _p(ids, ctypes.c_int32),
                                    _p(tw, ctypes.c_float), k, expert_begin, E, I, 1 if fp4 else 0,
                                    _p(w13, ctypes.c_uint8), s13.ctypes.data, _p(w2, ctypes.c_uint8),
                                    s2.ctypes.data, int(down_act_group), _p(out, ctypes.c_uint16),
                                    _p(qh, ctypes.c_uint8), _p(sh, ctypes.c_float), _p(y2, ctypes.c_double))
    if rc:
        raise ValueError("orc_fused_moe_recipe failed: %d" % rc)
    if not intermediates:
        return out
    fl = ids.ravel()
    Pl = int(np.count_nonzero((fl >= expert_begin) & (fl < expert_begin + E)))
    return out, dict(qh=qh[:Pl], sh=sh[:Pl], y2=y2[:Pl])


def swiglu(gate, up) -> np.ndarray:
    """h = silu(gate) * up (fp64), rounded once to fp32 -- the oracle's SwiGLU step."""
    g = _c(np.ravel(gate), np.float64)
    u = _c(np.ravel(up), np.float64)
    assert g.shape == u.shape
    h = np.empty(g.size, np.float32)
    lib().orc_swiglu(_p(g, ctypes.c_double), _p(u, ctypes.c_double), g.size, _p(h, ctypes.c_float))
    return h.reshape(np.shape(gate))


def quantize_f32(x: np.ndarray):
    x = _c(x, np.float32)
    M, K = x.shape
    codes = np.empty((M, K), np.uint8)
    scales = np.empty((M, K // 128), np.float32)
    lib().orc_quantize_rows_f32(_p(x, ctypes.c_float), M, K, _p(codes, ctypes.c_uint8),
                                _p(scales, ctypes.c_float))
    return codes, scales


def moe_align(topk_ids: np.ndarray, expert_begin: int, num_local_experts: int, block_m: int):
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    F = T * k
    E = num_local_experts
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sorted_ids = np.full(max(F, 1), -7, np.int32)
    src2dst = np.full(max(F, 1), -7, np.int32)
    nb_max = (F + block_m - 1) // block_m + E
    bexp = np.full(max(nb_max, 1), -7, np.int32)
    brow = np.full(max(nb_max, 1), -7, np.int32)
    nb = np.zeros(1, np.int32)
    rc = lib().orc_moe_align(_p(ids, ctypes.c_int32), T, k, expert_begin, E, block_m,
                             _p(counts, ctypes.c_int32), _p(offsets, ctypes.c_int32),
                             _p(sorted_ids, ctypes.c_int32), _p(src2dst, ctypes.c_int32),
                             _p(bexp, ctypes.c_int32), _p(brow, ctypes.c_int32),
                             _p(nb, ctypes.c_int32))
    if rc:
        raise ValueError("orc_moe_align failed: %d" % rc)
    P = int(offsets[E])
    n = int(nb[0])
    return dict(counts=counts, offsets=offsets, sorted_pair_ids=sorted_ids[:P],
                src2dst=src2dst[:F], block_expert=bexp[:n], block_row=brow[:n], num_blocks=n)


def gemm_f64(a, sa, w, sw) -> np.ndarray:
    a = _c(a, np.uint8)
    sa = _c(sa, np.float32)
    w = _c(w, np.uint8)
    sw = _c(sw, np.float32)
    M, K = a.shape
    N = w.shape[0]
    assert w.shape == (N, K // 2) and sa.shape == (M, K // 128) and sw.shape == (N, K // 128)
    y = np.empty((M, N), np.float64)
    lib().orc_gemm_f64(_p(a, ctypes.c_uint8), _p(sa, ctypes.c_float), M, K, _p(w, ctypes.c_uint8),
                       _p(sw, ctypes.c_float), N, _p(y, ctypes.c_double))
    return y


def gemm_bf16(a, sa, w, sw) -> np.ndarray:
    a = _c(a, np.uint8)
    sa = _c(sa, np.float32)
    w = _c(w, np.uint8)
    sw = _c(sw, np.float32)
    M, K = a.shape
    N = w.shape[0]
    assert w.shape == (N, K // 2) and sa.shape == (M, K // 128) and sw.shape == (N, K // 128)
    out = np.empty((M, N), np.uint16)
    lib().orc_gemm_bf16(_p(a, ctypes.c_uint8), _p(sa, ctypes.c_float), M, K, _p(w, ctypes.c_uint8),
                        _p(sw, ctypes.c_float), N, _p(out, ctypes.c_uint16))
    return out


def gemm_fp4_f64(a, sa, w, sw) -> np.ndarray:
    """codes [M, K] x fp4 e2m1 [N, K/2] with UE8M0 scales sw [N, K/32] -> fp64 [M, N]."""
    a = _c(a, np.uint8)
    sa = _c(sa, np.float32)
    w = _c(w, np.uint8)
    sw = _c(sw, np.uint8)
    M, K = a.shape
    N = w.shape[0]
    assert w.shape == (N, K // 2) and sa.shape == (M, K // 128) and sw.shape == (N, K // 32)
    y = np.empty((M, N), np.float64)
    lib().orc_gemm_fp4_f64(_p(a, ctypes.c_uint8), _p(sa, ctypes.c_float), M, K,
                           _p(w, ctypes.c_uint8), _p(sw, ctypes.c_uint8), N, _p(y, ctypes.c_double))
    return y


def fused_moe_fp4(hidden_bits, topk_ids, topk_weights, expert_begin, num_local_experts,
                  w13, s13, w2, s2, intermediates: bool = False):
    """The forward on fp4 weights: w13 [E, 2I, H/2] / w2 [E, H, I/2] e2m1
    nibbles, s13 [E, 2I, H/32] / s2 [E, H, I/32] UE8M0 bytes."""
    return fused_moe(hidden_bits, topk_ids, topk_weights, expert_begin, num_local_experts,
                     w13, s13, w2, s2, intermediates, fp4=True)


def fused_moe(hidden_bits, topk_ids, topk_weights, expert_begin, num_local_experts,
              w13, s13, w2, s2, intermediates: bool = False, fp4: bool = False):
    """The whole forward.  Returns bf16 bits [T, H]; with ``intermediates``
    also a dict of qh [P, I] codes, sh [P, I/128] scales and y2 [P, H] (fp64),
    in permuted pair order."""
    x = _c(hidden_bits, np.uint16)
    ids = _c(topk_ids, np.int32)
    tw = _c(topk_weights, np.float32)
    sdt, sblk = (np.uint8, 32) if fp4 else (np.float32, 128)
    w13 = _c(w13, np.uint8)
    s13 = _c(s13, sdt)
    w2 = _c(w2, np.uint8)
    s2 = _c(s2, sdt)
    T, H = x.shape
    k = ids.shape[1]
    E = num_local_experts
    I = w2.shape[2] * 2
    assert w13.shape == (E, 2 * I, H // 2) and s13.shape == (E, 2 * I, H // sblk)
    assert w2.shape == (E, H, I // 2) and s2.shape == (E, H, I // sblk)
    assert ids.shape == (T, k) and tw.shape == (T, k)
    out = np.empty((T, H), np.uint16)
    qh = sh = y2 = None
    if intermediates:
        P = T * k
        qh = np.zeros((max(P, 1), I), np.uint8)
        sh = np.zeros((max(P, 1), I // 128), np.float32)
        y2 = np.zeros((max(P, 1), H), np.float64)
    sct = ctypes.c_uint8 if fp4 else ctypes.c_float
    fn = lib().orc_fused_moe_fp4 if fp4 else lib().orc_fused_moe
    rc = fn(_p(x, ctypes.c_uint16), T, H, _p(ids, ctypes.c_int32),
            _p(tw, ctypes.c_float), k, expert_begin, E, I,
            _p(w13, ctypes.c_uint8), _p(s13, sct),
            _p(w2, ctypes.c_uint8), _p(s2, sct),
            _p(out, ctypes.c_uint16), _p(qh, ctypes.c_uint8),
            _p(sh, ctypes.c_float), _p(y2, ctypes.c_double))
    if rc:
        raise ValueError("orc fused forward failed: %d" % rc)
    if not intermediates:
        return out
    ids_flat = ids.ravel()
    P = int(np.count_nonzero((ids_flat >= expert_begin) & (ids_flat < expert_begin + E)))
    return out, dict(qh=qh[:P], sh=sh[:P], y2=y2[:P])
