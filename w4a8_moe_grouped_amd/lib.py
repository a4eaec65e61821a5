"""Thin Python binding of libw4a8 (include/w4a8.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream, every step of the computation runs in the library's HIP kernels.
There is no fallback: if libw4a8.so is missing or the call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libw4a8.so")

W4A8_OK = 0
GROUP = 128
EXPORTS = ("w4a8_version", "w4a8_status_string", "w4a8_quantize_act", "w4a8_gemm",
           "w4a8_moe_align", "w4a8_fused_moe", "w4a8_fused_moe_workspace_layout",
           "w4a8_fused_moe_stage_events", "w4a8_prepack_weights", "w4a8_prepacked_scale_count",
           "w4a8_fused_moe_prepacked", "w4a8_prepack_weights_fp4", "w4a8_fused_moe_fp4_prepacked",
           "w4a8_prepack_weights_bf16_scales", "w4a8_fused_moe_prepacked_static",
           "w4a8_fused_moe_recipe", "w4a8_fused_moe_prepacked_noalloc", "w4a8_fused_moe_bounded",
           "w4a8_fused_moe_persistent")

_lock = threading.Lock()
_lib = None


class W4A8Error(RuntimeError):
    pass


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libw4a8.so (built by ``python -m w4a8_moe_grouped_amd.build``)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise W4A8Error("libw4a8.so not built at %s (run python -m w4a8_moe_grouped_amd.build)" % p)
        L = ctypes.CDLL(p)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)
        L.w4a8_version.restype = ctypes.c_int
        L.w4a8_version.argtypes = []
        L.w4a8_status_string.restype = ctypes.c_char_p
        L.w4a8_status_string.argtypes = [ctypes.c_int]
        L.w4a8_quantize_act.restype = ctypes.c_int
        L.w4a8_quantize_act.argtypes = [vp, i64, i64, i64, vp, vp, vp]
        L.w4a8_gemm.restype = ctypes.c_int
        L.w4a8_gemm.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp, sz, vp]
        L.w4a8_moe_align.restype = ctypes.c_int
        L.w4a8_moe_align.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp,
                                     vp, sz, vp]
        L.w4a8_fused_moe.restype = ctypes.c_int
        L.w4a8_fused_moe.argtypes = [vp, i64, i64, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp,
                                     vp, vp, sz, vp]
        L.w4a8_fused_moe_prepacked.restype = ctypes.c_int
        L.w4a8_fused_moe_prepacked.argtypes = L.w4a8_fused_moe.argtypes
        L.w4a8_prepack_weights.restype = ctypes.c_int
        L.w4a8_prepack_weights.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
        L.w4a8_fused_moe_fp4_prepacked.restype = ctypes.c_int
        L.w4a8_fused_moe_fp4_prepacked.argtypes = L.w4a8_fused_moe.argtypes
        L.w4a8_prepack_weights_fp4.restype = ctypes.c_int
        L.w4a8_prepack_weights_fp4.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, vp, vp, vp]
        L.w4a8_fused_moe_prepacked_static.restype = ctypes.c_int
        L.w4a8_fused_moe_prepacked_static.argtypes = L.w4a8_fused_moe.argtypes[:13] + [vp, vp] + \
            L.w4a8_fused_moe.argtypes[13:]
        L.w4a8_fused_moe_recipe.restype = ctypes.c_int
        L.w4a8_fused_moe_recipe.argtypes = [vp, i64, i64, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                            vp, vp, vp, vp, ctypes.c_int, vp, vp, sz, vp]
        L.w4a8_fused_moe_persistent.restype = ctypes.c_int
        L.w4a8_fused_moe_persistent.argtypes = [vp, i64, i64, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                                vp, vp, vp, vp, vp, vp, sz, vp]
        L.w4a8_fused_moe_bounded.restype = ctypes.c_int
        L.w4a8_fused_moe_bounded.argtypes = [vp, i64, i64, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                             vp, vp, vp, vp, i64, vp, vp, vp, sz, vp]
        L.w4a8_fused_moe_prepacked_noalloc.restype = ctypes.c_int
        L.w4a8_fused_moe_prepacked_noalloc.argtypes = L.w4a8_fused_moe.argtypes[:14] + [vp]
        L.w4a8_prepack_weights_bf16_scales.restype = ctypes.c_int
        L.w4a8_prepack_weights_bf16_scales.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
        L.w4a8_prepacked_scale_count.restype = ctypes.c_int64
        L.w4a8_prepacked_scale_count.argtypes = [i64, i64, i64]
        L.w4a8_fused_moe_workspace_layout.restype = ctypes.c_int
        L.w4a8_fused_moe_workspace_layout.argtypes = [i64, i64, i64, i64, i64,
                                                      ctypes.POINTER(ctypes.c_size_t), ctypes.c_int,
                                                      ctypes.POINTER(ctypes.c_int64)]
        L.w4a8_fused_moe_stage_events.restype = ctypes.c_int
        L.w4a8_fused_moe_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
        if path is None:
            _lib = L
        return L


def _check(rc: int, what: str):
    if rc != W4A8_OK:
        msg = load().w4a8_status_string(rc).decode()
        raise W4A8Error("%s failed: %s (%d)" % (what, msg, rc))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise W4A8Error("all tensors must be on the GPU")


# ---- workspace sizes (host-only queries) ----------------------------------------

def gemm_workspace_bytes(M: int, K: int, N: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().w4a8_gemm(None, None, M, K, None, None, N, None, None, ctypes.byref(n), None),
           "w4a8_gemm(query)")
    return n.value


def align_workspace_bytes(T: int, topk: int, num_local_experts: int, block_m: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().w4a8_moe_align(None, T, topk, 0, num_local_experts, block_m, None, None, None,
                                 None, None, None, None, None, ctypes.byref(n), None),
           "w4a8_moe_align(query)")
    return n.value


def fused_moe_workspace_bytes(T: int, H: int, topk: int, num_local_experts: int, I: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().w4a8_fused_moe(None, T, H, None, None, topk, 0, num_local_experts, I, None, None,
                                 None, None, None, None, ctypes.byref(n), None),
           "w4a8_fused_moe(query)")
    return n.value


LAYOUT_KEYS = ("counts", "offsets", "sorted_pair_ids", "src2dst", "block_expert", "block_row",
               "num_blocks", "qa16", "qa_side", "qh", "qh_side", "y2", "block_expert2", "block_row2",
               "num_blocks2", "block_row3", "num_blocks3", "path")


def fused_moe_workspace_layout(T: int, H: int, topk: int, num_local_experts: int, I: int):
    """Byte offsets of the intermediates inside the fused forward's workspace."""
    offs = (ctypes.c_size_t * 18)()
    bm = ctypes.c_int64(0)
    _check(load().w4a8_fused_moe_workspace_layout(T, H, topk, num_local_experts, I, offs, 18,
                                                  ctypes.byref(bm)),
           "w4a8_fused_moe_workspace_layout")
    d = dict(zip(LAYOUT_KEYS, [int(o) for o in offs]))
    d["block_m"] = int(bm.value)
    d["two_lists"] = d["num_blocks2"] != 0
    d["device_path"] = d["path"] != 0  # the path is chosen on the device
    return d


# ---- exports ----------------------------------------------------------------------

def prepack_weights(w: torch.Tensor, w_scales: torch.Tensor):
    """int4 [E, N, K/2] + fp32 or bf16 scales [E, N, K/128] -> (packed uint8
    [E, N*K/2], packed fp32 scales [E, count/E]) in the layout of w4a8_prepack_weights."""
    _need_cuda(w, w_scales)
    if w.dim() != 3 or w.dtype != torch.uint8 or not w.is_contiguous() or not w_scales.is_contiguous():
        raise W4A8Error("w must be a contiguous uint8 [E, N, K/2] tensor")
    E, N, K2 = w.shape
    K = 2 * K2
    cnt = int(load().w4a8_prepacked_scale_count(E, N, K))
    if cnt < 0 or w_scales.shape != (E, N, K // GROUP) or \
            w_scales.dtype not in (torch.float32, torch.bfloat16):
        raise W4A8Error("bad weight / scale shapes")
    wp = torch.empty((E, N * K2), dtype=torch.uint8, device=w.device)
    sp = torch.empty((E, cnt // E), dtype=torch.float32, device=w.device)
    if w_scales.dtype == torch.bfloat16:  # a checkpoint's bf16 scales, widened exactly
        fn, name = load().w4a8_prepack_weights_bf16_scales, "w4a8_prepack_weights_bf16_scales"
    else:
        fn, name = load().w4a8_prepack_weights, "w4a8_prepack_weights"
    _check(fn(_ptr(w), _ptr(w_scales), E, N, K, _ptr(wp), _ptr(sp), _stream(w.device)), name)
    return wp, sp


FP4_GATE_UP, FP4_DOWN = 0, 1


def prepack_weights_fp4(w: torch.Tensor, w_scales: torch.Tensor, role: int):
    """fp4 e2m1 [E, N, K/2] + UE8M0 uint8 scales [E, N, K/32] -> (packed
    uint8 [E, N*K/2], packed scale dwords int32 [E, count/E]) in the layout of
    w4a8_prepack_weights_fp4 (role FP4_GATE_UP for w13, FP4_DOWN for w2)."""
    _need_cuda(w, w_scales)
    if w.dim() != 3 or w.dtype != torch.uint8 or not w.is_contiguous() or not w_scales.is_contiguous():
        raise W4A8Error("w must be a contiguous uint8 [E, N, K/2] tensor")
    E, N, K2 = w.shape
    K = 2 * K2
    cnt = int(load().w4a8_prepacked_scale_count(E, N, K))
    if cnt < 0 or w_scales.shape != (E, N, K // 32) or w_scales.dtype != torch.uint8:
        raise W4A8Error("bad weight / scale shapes")
    wp = torch.empty((E, N * K2), dtype=torch.uint8, device=w.device)
    sp = torch.empty((E, cnt // E), dtype=torch.int32, device=w.device)
    _check(load().w4a8_prepack_weights_fp4(_ptr(w), _ptr(w_scales), E, N, K, int(role), _ptr(wp),
                                           _ptr(sp), _stream(w.device)), "w4a8_prepack_weights_fp4")
    return wp, sp


def fused_moe_fp4(hidden: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                  expert_begin: int, num_local_experts: int, I: int, prepacked: tuple,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """The fused forward on fp4 weights; prepacked = (w13p, s13p, w2p, s2p)
    from prepack_weights_fp4 (w13 with FP4_GATE_UP, w2 with FP4_DOWN)."""
    w13p, s13p, w2p, s2p = prepacked
    _need_cuda(hidden, topk_ids, topk_weights, w13p, s13p, w2p, s2p)
    T, H = hidden.shape
    k = topk_ids.shape[1]
    E = num_local_experts
    assert hidden.dtype == torch.bfloat16 and topk_ids.dtype == torch.int32 \
        and topk_weights.dtype == torch.float32
    assert topk_ids.shape == (T, k) and topk_weights.shape == (T, k)
    assert w13p.numel() == E * 2 * I * H // 2 and w2p.numel() == E * H * I // 2
    assert s13p.numel() == load().w4a8_prepacked_scale_count(E, 2 * I, H)
    assert s2p.numel() == load().w4a8_prepacked_scale_count(E, H, I)
    for t in (hidden, topk_ids, topk_weights, w13p, s13p, w2p, s2p):
        assert t.is_contiguous()
    out = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=hidden.device)
    if workspace is None:
        need = fused_moe_workspace_bytes(T, H, k, E, I)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(load().w4a8_fused_moe_fp4_prepacked(
        _ptr(hidden), T, H, _ptr(topk_ids), _ptr(topk_weights), k, expert_begin, E, I,
        _ptr(w13p), _ptr(s13p), _ptr(w2p), _ptr(s2p), _ptr(out), _ptr(workspace),
        ctypes.byref(n), _stream(hidden.device)), "w4a8_fused_moe_fp4_prepacked")
    return out


def fused_moe_noalloc(hidden: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                      expert_begin: int, num_local_experts: int, I: int, prepacked: tuple,
                      out: Optional[torch.Tensor] = None):
    """w4a8_fused_moe_prepacked_noalloc: the fused forward on prepacked int4
    weights (w13p, s13p, w2p, s2p) with no workspace argument (the library's
    own device array holds the intermediates)."""
    w13p, s13p, w2p, s2p = prepacked
    _need_cuda(hidden, topk_ids, topk_weights, w13p, s13p, w2p, s2p)
    T, H = hidden.shape
    k = topk_ids.shape[1]
    E = num_local_experts
    assert hidden.dtype == torch.bfloat16 and topk_ids.dtype == torch.int32 \
        and topk_weights.dtype == torch.float32
    assert topk_ids.shape == (T, k) and topk_weights.shape == (T, k)
    assert w13p.numel() == E * 2 * I * H // 2 and w2p.numel() == E * H * I // 2
    assert s13p.numel() == load().w4a8_prepacked_scale_count(E, 2 * I, H)
    assert s2p.numel() == load().w4a8_prepacked_scale_count(E, H, I)
    for t in (hidden, topk_ids, topk_weights, w13p, s13p, w2p, s2p):
        assert t.is_contiguous()
    out = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=hidden.device)
    _check(load().w4a8_fused_moe_prepacked_noalloc(
        _ptr(hidden), T, H, _ptr(topk_ids), _ptr(topk_weights), k, expert_begin, E, I,
        _ptr(w13p), _ptr(s13p), _ptr(w2p), _ptr(s2p), _ptr(out), _stream(hidden.device)),
        "w4a8_fused_moe_prepacked_noalloc")
    return out


WEIGHTS_INT4, WEIGHTS_INT4_PACKED, WEIGHTS_FP4_PACKED = 0, 1, 2


def fused_moe_bounded_workspace_bytes(T: int, H: int, topk: int, num_local_experts: int, I: int,
                                      max_local_pairs: int, weight_format: int = WEIGHTS_INT4_PACKED) -> int:
    n = ctypes.c_size_t(0)
    _check(load().w4a8_fused_moe_bounded(None, T, H, None, None, topk, 0, num_local_experts, I,
                                         int(weight_format), None, None, None, None, int(max_local_pairs),
                                         None, None, None, ctypes.byref(n), None),
           "w4a8_fused_moe_bounded(query)")
    return n.value


def fused_moe_bounded(hidden: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                      expert_begin: int, num_local_experts: int, I: int, weights: tuple,
                      weight_format: int, max_local_pairs: int, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      local_pairs: Optional[torch.Tensor] = None):
    """w4a8_fused_moe_bounded: the fused forward with per-pair buffers sized
    for max_local_pairs local pairs.  weights = (w13, s13, w2, s2) in the
    layout weight_format names.  Returns (out, local_pairs), the latter a
    two-element int32 device tensor the call writes with the local pair count
    (out is all +0 when it exceeds the bound) and the path (1: block-tiled
    kernels, 0: few-rows kernels)."""
    w13, s13, w2, s2 = weights
    _need_cuda(hidden, topk_ids, topk_weights, w13, s13, w2, s2)
    T, H = hidden.shape
    k = topk_ids.shape[1]
    E = num_local_experts
    assert hidden.dtype == torch.bfloat16 and topk_ids.dtype == torch.int32 \
        and topk_weights.dtype == torch.float32
    assert topk_ids.shape == (T, k) and topk_weights.shape == (T, k)
    assert w13.numel() == E * 2 * I * H // 2 and w2.numel() == E * H * I // 2
    for t in (hidden, topk_ids, topk_weights, w13, s13, w2, s2):
        assert t.is_contiguous()
    out = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=hidden.device)
    if local_pairs is None:
        local_pairs = torch.full((2,), -1, dtype=torch.int32, device=hidden.device)
    assert local_pairs.is_cuda and local_pairs.dtype == torch.int32 and local_pairs.numel() >= 2
    if workspace is None:
        need = fused_moe_bounded_workspace_bytes(T, H, k, E, I, max_local_pairs, weight_format)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(load().w4a8_fused_moe_bounded(
        _ptr(hidden), T, H, _ptr(topk_ids), _ptr(topk_weights), k, expert_begin, E, I,
        int(weight_format), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), int(max_local_pairs),
        _ptr(local_pairs), _ptr(out), _ptr(workspace), ctypes.byref(n), _stream(hidden.device)),
        "w4a8_fused_moe_bounded")
    return out, local_pairs


def fused_moe_persistent_workspace_bytes(T: int, H: int, topk: int, num_local_experts: int, I: int,
                                         weight_format: int = WEIGHTS_INT4_PACKED) -> int:
    n = ctypes.c_size_t(0)
    _check(load().w4a8_fused_moe_persistent(None, T, H, None, None, topk, 0, num_local_experts, I,
                                            int(weight_format), None, None, None, None, None, None,
                                            ctypes.byref(n), None),
           "w4a8_fused_moe_persistent(query)")
    return n.value


def fused_moe_persistent(hidden: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                         expert_begin: int, num_local_experts: int, I: int, weights: tuple,
                         weight_format: int, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w4a8_fused_moe_persistent: the align launch, then gate_up, down and
    the combine in one cooperative launch.  weights = (w13, s13, w2, s2) in
    the layout weight_format names."""
    w13, s13, w2, s2 = weights
    _need_cuda(hidden, topk_ids, topk_weights, w13, s13, w2, s2)
    T, H = hidden.shape
    k = topk_ids.shape[1]
    E = num_local_experts
    assert hidden.dtype == torch.bfloat16 and topk_ids.dtype == torch.int32 \
        and topk_weights.dtype == torch.float32
    assert topk_ids.shape == (T, k) and topk_weights.shape == (T, k)
    assert w13.numel() == E * 2 * I * H // 2 and w2.numel() == E * H * I // 2
    for t in (hidden, topk_ids, topk_weights, w13, s13, w2, s2):
        assert t.is_contiguous()
    out = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=hidden.device)
    if workspace is None:
        need = fused_moe_persistent_workspace_bytes(T, H, k, E, I, weight_format)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(load().w4a8_fused_moe_persistent(
        _ptr(hidden), T, H, _ptr(topk_ids), _ptr(topk_weights), k, expert_begin, E, I,
        int(weight_format), _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), _ptr(out), _ptr(workspace),
        ctypes.byref(n), _stream(hidden.device)),
        "w4a8_fused_moe_persistent")
    return out


def fused_moe_recipe(hidden: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                     expert_begin: int, num_local_experts: int, I: int, prepacked: tuple,
                     weight_format: int, down_act_group: int, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """The fused forward with the down GEMM's input quantised per
    down_act_group (128, 64 or 32) K; prepacked = (w13p, s13p, w2p, s2p) from
    prepack_weights (WEIGHTS_INT4_PACKED) or prepack_weights_fp4
    (WEIGHTS_FP4_PACKED)."""
    w13p, s13p, w2p, s2p = prepacked
    _need_cuda(hidden, topk_ids, topk_weights, w13p, s13p, w2p, s2p)
    T, H = hidden.shape
    k = topk_ids.shape[1]
    E = num_local_experts
    assert hidden.dtype == torch.bfloat16 and topk_ids.dtype == torch.int32 \
        and topk_weights.dtype == torch.float32
    assert w13p.numel() == E * 2 * I * H // 2 and w2p.numel() == E * H * I // 2
    for t in (hidden, topk_ids, topk_weights, w13p, s13p, w2p, s2p):
        assert t.is_contiguous()
    out = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=hidden.device)
    if workspace is None:
        need = fused_moe_workspace_bytes(T, H, k, E, I)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(load().w4a8_fused_moe_recipe(
        _ptr(hidden), T, H, _ptr(topk_ids), _ptr(topk_weights), k, expert_begin, E, I,
        int(weight_format), _ptr(w13p), _ptr(s13p), _ptr(w2p), _ptr(s2p), int(down_act_group),
        _ptr(out), _ptr(workspace), ctypes.byref(n), _stream(hidden.device)), "w4a8_fused_moe_recipe")
    return out


def quantize_act(x: torch.Tensor, out_q: Optional[torch.Tensor] = None,
                 out_scales: Optional[torch.Tensor] = None):
    """bf16 [M, K] -> (uint8 e4m3 codes [M, K], fp32 scales [M, K/128])."""
    _need_cuda(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise W4A8Error("x must be a 2-D bf16 tensor with unit column stride")
    M, K = x.shape
    q = out_q if out_q is not None else torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = out_scales if out_scales is not None else \
        torch.empty((M, K // GROUP), dtype=torch.float32, device=x.device)
    _check(load().w4a8_quantize_act(_ptr(x), M, K, x.stride(0), _ptr(q), _ptr(s), _stream(x.device)),
           "w4a8_quantize_act")
    return q, s


def gemm(a_q: torch.Tensor, a_scales: torch.Tensor, w: torch.Tensor, w_scales: torch.Tensor,
         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """codes [M, K] x packed int4 [N, K/2] -> bf16 [M, N]."""
    _need_cuda(a_q, a_scales, w, w_scales)
    M, K = a_q.shape
    N = w.shape[0]
    assert w.shape == (N, K // 2) and a_scales.shape == (M, K // GROUP) \
        and w_scales.shape == (N, K // GROUP)
    out = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    need = gemm_workspace_bytes(M, K, N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=a_q.device)
    n = ctypes.c_size_t(workspace.numel())
    _check(load().w4a8_gemm(_ptr(a_q), _ptr(a_scales), M, K, _ptr(w), _ptr(w_scales), N,
                            _ptr(out), _ptr(workspace), ctypes.byref(n), _stream(a_q.device)),
           "w4a8_gemm")
    return out


def moe_align(topk_ids: torch.Tensor, expert_begin: int, num_local_experts: int, block_m: int):
    """Routing permutation; returns a dict of device tensors (see w4a8.h)."""
    _need_cuda(topk_ids)
    T, k = topk_ids.shape
    F = T * k
    E = num_local_experts
    dev = topk_ids.device
    nb_max = (F + block_m - 1) // block_m + E
    o = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
             offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
             sorted_pair_ids=torch.empty(max(F, 1), dtype=torch.int32, device=dev),
             src2dst=torch.empty(max(F, 1), dtype=torch.int32, device=dev),
             block_expert=torch.empty(max(nb_max, 1), dtype=torch.int32, device=dev),
             block_row=torch.empty(max(nb_max, 1), dtype=torch.int32, device=dev),
             num_blocks=torch.empty(1, dtype=torch.int32, device=dev))
    need = align_workspace_bytes(T, k, E, block_m)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    n = ctypes.c_size_t(ws.numel())
    _check(load().w4a8_moe_align(_ptr(topk_ids), T, k, expert_begin, E, block_m,
                                 _ptr(o["counts"]), _ptr(o["offsets"]), _ptr(o["sorted_pair_ids"]),
                                 _ptr(o["src2dst"]), _ptr(o["block_expert"]), _ptr(o["block_row"]),
                                 _ptr(o["num_blocks"]), _ptr(ws), ctypes.byref(n), _stream(dev)),
           "w4a8_moe_align")
    return o


STAGES = ("align", "quant", "gate_up", "down", "combine")


# Timing-only events skip the system-scope release fence (a cache writeback
# that otherwise lands inside the measured span and inflates it by a few us).
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _hip_timing_api():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def _timing_event(hip):
    h = ctypes.c_void_p()
    if hip.hipEventCreateWithFlags(ctypes.byref(h), _HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
        raise W4A8Error("hipEventCreateWithFlags failed")
    return h


class StageTimer:
    """HIP events around the five stages of the next fused_moe call(s).

    Uses the HIP runtime's own event API (through ctypes) so the events sit on
    the very stream the library launches on."""

    def __init__(self):
        self.hip = _hip_timing_api()
        self.ev = (ctypes.c_void_p * 6)()
        for i in range(6):
            self.ev[i] = _timing_event(self.hip)

    def arm(self):
        _check(load().w4a8_fused_moe_stage_events(self.ev, 6), "w4a8_fused_moe_stage_events")

    def read_ms(self):
        """Per-stage milliseconds of the last armed call (synchronises on its last event)."""
        self.hip.hipEventSynchronize(self.ev[5])
        out = []
        for i in range(5):
            ms = ctypes.c_float()
            self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[i + 1])
            out.append(ms.value)
        return dict(zip(STAGES, out))

    def close(self):
        for i in range(6):
            self.hip.hipEventDestroy(self.ev[i])


class SpanTimer:
    """HIP events around one stage (events `first` -> `last` of the stage
    hook, see STAGES) of each of the next `n` fused_moe calls, one event pair
    per call, recorded on the library's stream; the other hook slots stay
    empty so a call records only two events."""

    def __init__(self, first: int, last: int, n: int):
        if not (0 <= first < last <= 5) or n < 1:
            raise W4A8Error("bad span")
        self.hip = _hip_timing_api()
        self.first, self.last, self.n = first, last, n
        self.ev = [_timing_event(self.hip) for _ in range(2 * n)]
        self.slots = []
        for j in range(n):
            arr = (ctypes.c_void_p * 6)()
            arr[first] = self.ev[2 * j]
            arr[last] = self.ev[2 * j + 1]
            self.slots.append(arr)

    def arm(self, j: int):
        _check(load().w4a8_fused_moe_stage_events(self.slots[j], 6), "w4a8_fused_moe_stage_events")

    def read_ms(self):
        """Milliseconds of the span in each of the n calls (synchronises)."""
        out = []
        for j in range(self.n):
            self.hip.hipEventSynchronize(self.ev[2 * j + 1])
            ms = ctypes.c_float()
            self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[2 * j], self.ev[2 * j + 1])
            out.append(ms.value)
        return out

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


def fused_moe(hidden: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
              expert_begin: int, num_local_experts: int, w13: torch.Tensor, s13: torch.Tensor,
              w2: torch.Tensor, s2: torch.Tensor, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, prepacked: Optional[tuple] = None,
              a1_scale: Optional[torch.Tensor] = None, a2_scale: Optional[torch.Tensor] = None):
    """The fused forward; bf16 [T, H] out.  w13/s13/w2/s2 are the canonical
    weights (they give the shapes); with prepacked = (w13p, s13p, w2p, s2p)
    from prepack_weights, w4a8_fused_moe_prepacked runs on those instead, and
    with static activation scales (one-element fp32 device tensors, either may
    be None = dynamic) w4a8_fused_moe_prepacked_static."""
    _need_cuda(hidden, topk_ids, topk_weights, w13, s13, w2, s2)
    T, H = hidden.shape
    k = topk_ids.shape[1]
    E = num_local_experts
    I = w2.shape[2] * 2
    assert hidden.dtype == torch.bfloat16 and topk_ids.dtype == torch.int32 \
        and topk_weights.dtype == torch.float32
    assert w13.shape == (E, 2 * I, H // 2) and s13.shape == (E, 2 * I, H // GROUP)
    assert w2.shape == (E, H, I // 2) and s2.shape == (E, H, I // GROUP)
    assert topk_ids.shape == (T, k) and topk_weights.shape == (T, k)
    for t in (hidden, topk_ids, topk_weights, w13, s13, w2, s2):
        assert t.is_contiguous()
    out = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=hidden.device)
    if workspace is None:
        need = fused_moe_workspace_bytes(T, H, k, E, I)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=hidden.device)
    n = ctypes.c_size_t(workspace.numel())
    if prepacked is not None:
        w13p, s13p, w2p, s2p = prepacked
        _need_cuda(w13p, s13p, w2p, s2p)
        assert w13p.numel() == w13.numel() and w2p.numel() == w2.numel()
        assert s13p.numel() == load().w4a8_prepacked_scale_count(E, 2 * I, H)
        assert s2p.numel() == load().w4a8_prepacked_scale_count(E, H, I)
        fn, name = load().w4a8_fused_moe_prepacked, "w4a8_fused_moe_prepacked"
        ws = (w13p, s13p, w2p, s2p)
        if a1_scale is not None or a2_scale is not None:
            for t in (a1_scale, a2_scale):
                assert t is None or (t.is_cuda and t.dtype == torch.float32 and t.numel() == 1)
            stat = (_ptr(a1_scale) if a1_scale is not None else None,
                    _ptr(a2_scale) if a2_scale is not None else None)
            _check(load().w4a8_fused_moe_prepacked_static(
                _ptr(hidden), T, H, _ptr(topk_ids), _ptr(topk_weights), k, expert_begin, E, I,
                _ptr(ws[0]), _ptr(ws[1]), _ptr(ws[2]), _ptr(ws[3]), stat[0], stat[1], _ptr(out),
                _ptr(workspace), ctypes.byref(n), _stream(hidden.device)), "w4a8_fused_moe_prepacked_static")
            return out
    else:
        assert a1_scale is None and a2_scale is None, "static scales need prepacked weights"
        fn, name = load().w4a8_fused_moe, "w4a8_fused_moe"
        ws = (w13, s13, w2, s2)
    _check(fn(_ptr(hidden), T, H, _ptr(topk_ids), _ptr(topk_weights), k, expert_begin, E, I,
              _ptr(ws[0]), _ptr(ws[1]), _ptr(ws[2]), _ptr(ws[3]), _ptr(out), _ptr(workspace),
              ctypes.byref(n), _stream(hidden.device)), name)
    return out
