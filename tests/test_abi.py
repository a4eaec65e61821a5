"""Host-only checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/w4a8.h declares, answer
workspace queries as a pure function of the shapes, and reject bad arguments
with the documented status before any HIP call is made.
"""
import ctypes
import os
import re

import pytest

from w4a8_moe_grouped_amd import lib as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
BOGUS = ctypes.c_void_p(0x1000)  # 16-byte aligned, never dereferenced on these paths
MISALIGNED = ctypes.c_void_p(0x1004)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(w4.LIB_PATH):
        from w4a8_moe_grouped_amd import build
        build.build()
    return w4.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(w4a8_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(w4.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.w4a8_version() >= 1
    for rc in range(5):
        assert L.w4a8_status_string(rc)
    assert L.w4a8_status_string(99) == b"unknown status"


def test_workspace_queries_are_pure_functions_of_shape(L):
    a = w4.fused_moe_workspace_bytes(64, 7168, 8, 32, 2048)
    assert a == w4.fused_moe_workspace_bytes(64, 7168, 8, 32, 2048) and a > 0
    assert w4.fused_moe_workspace_bytes(128, 7168, 8, 32, 2048) > a
    assert w4.gemm_workspace_bytes(128, 7168, 2048) >= 128 * 7168
    assert w4.align_workspace_bytes(64, 8, 32, 16) > 0
    big = w4.align_workspace_bytes(32768, 8, 32, 64)
    assert big >= 64 * 32 * 4  # per-chunk histograms


def _fused(L, T=4, H=256, k=2, E=4, I=128, hidden=BOGUS, ids=BOGUS, wts=BOGUS, w13=BOGUS,
           ws=BOGUS, nbytes=None):
    n = ctypes.c_size_t(1 << 40 if nbytes is None else nbytes)
    return L.w4a8_fused_moe(hidden, T, H, ids, wts, k, 0, E, I, w13, BOGUS, BOGUS, BOGUS, BOGUS,
                            ws, ctypes.byref(n), None)


def test_fused_moe_rejects_bad_arguments(L):
    assert _fused(L, H=200) == UNSUPPORTED
    assert _fused(L, I=100) == UNSUPPORTED
    assert _fused(L, k=33) == UNSUPPORTED
    assert _fused(L, E=2000) == UNSUPPORTED
    assert _fused(L, T=-1) == INVALID
    assert _fused(L, H=0) == INVALID
    assert _fused(L, k=0) == INVALID
    assert _fused(L, E=0) == INVALID
    assert _fused(L, hidden=None) == INVALID
    assert _fused(L, w13=None) == INVALID
    assert _fused(L, hidden=MISALIGNED) == UNSUPPORTED
    assert _fused(L, ws=MISALIGNED) == UNSUPPORTED
    assert _fused(L, nbytes=16) == WORKSPACE
    # T == 0 is valid and launches nothing
    assert _fused(L, T=0) == OK


def test_quantize_rejects_bad_arguments(L):
    q = L.w4a8_quantize_act
    assert q(BOGUS, 4, 100, 100, BOGUS, BOGUS, None) == UNSUPPORTED
    assert q(BOGUS, 4, 128, 64, BOGUS, BOGUS, None) == INVALID     # ldx < K
    assert q(BOGUS, 4, 128, 132, BOGUS, BOGUS, None) == UNSUPPORTED  # ldx % 8
    assert q(None, 4, 128, 128, BOGUS, BOGUS, None) == INVALID
    assert q(BOGUS, -1, 128, 128, BOGUS, BOGUS, None) == INVALID
    assert q(MISALIGNED, 4, 128, 128, BOGUS, BOGUS, None) == UNSUPPORTED
    assert q(None, 0, 128, 128, None, None, None) == OK


def test_fused_moe_rejects_32bit_range_overflow(L):
    """Every operand a kernel reads through a buffer resource (32-bit extent
    and offsets) must stay below 2^32 bytes; validation returns before any
    launch (the pointers here are bogus and never touched)."""
    # T*topk*I = 262144 * 8 * 2048 = 2^32: the down GEMM's activation rows
    assert _fused(L, T=262144, H=128, k=8, E=32, I=2048) == UNSUPPORTED
    # T*H = 2^32: the gate_up operand
    assert _fused(L, T=1 << 19, H=8192, k=1, E=32, I=128) == UNSUPPORTED
    # one expert's w13 (I*H bytes) reaches 2^32
    assert _fused(L, T=1, H=65536, k=1, E=1, I=65536) == UNSUPPORTED
    # huge T: no int64 overflow in the checks
    assert _fused(L, T=1 << 61, H=128, k=32, E=1, I=128) == UNSUPPORTED


def test_gemm_rejects_32bit_range_overflow(L):
    n = ctypes.c_size_t(1 << 62)
    g = L.w4a8_gemm
    # M*K = 2^32
    assert g(BOGUS, BOGUS, 1 << 19, 8192, BOGUS, BOGUS, 16, BOGUS, BOGUS, ctypes.byref(n), None) == UNSUPPORTED
    # N*K/2 = 2^32
    assert g(BOGUS, BOGUS, 4, 8192, BOGUS, BOGUS, 1 << 20, BOGUS, BOGUS, ctypes.byref(n), None) == UNSUPPORTED
    assert g(BOGUS, BOGUS, 1 << 40, 128, BOGUS, BOGUS, 16, BOGUS, BOGUS, ctypes.byref(n), None) == UNSUPPORTED


def test_prepack_rejects_32bit_range_overflow(L):
    other = ctypes.c_void_p(0x2000)
    # one expert's weights N*K/2 = 2^32
    assert L.w4a8_prepack_weights(BOGUS, BOGUS, 1, 1 << 20, 8192, other, other, None) == UNSUPPORTED


def test_stage_events_arming_is_copied_and_consumed(L):
    """The handles are copied at arming; any fused call (here a size query)
    consumes the arming; arming rejects a bad count."""
    arr = (ctypes.c_void_p * 6)()
    assert L.w4a8_fused_moe_stage_events(arr, 5) == INVALID
    assert L.w4a8_fused_moe_stage_events(None, 6) == INVALID
    assert L.w4a8_fused_moe_stage_events(arr, 6) == OK
    del arr
    n = ctypes.c_size_t(0)
    assert L.w4a8_fused_moe(None, 4, 256, None, None, 2, 0, 4, 128, None, None, None, None, None,
                            None, ctypes.byref(n), None) == OK
    assert L.w4a8_fused_moe_stage_events(None, 0) == OK


def test_gemm_rejects_bad_arguments(L):
    n = ctypes.c_size_t(1 << 40)
    g = L.w4a8_gemm
    assert g(BOGUS, BOGUS, 4, 100, BOGUS, BOGUS, 16, BOGUS, BOGUS, ctypes.byref(n), None) == UNSUPPORTED
    assert g(BOGUS, BOGUS, 4, 128, BOGUS, BOGUS, 0, BOGUS, BOGUS, ctypes.byref(n), None) == INVALID
    assert g(None, BOGUS, 4, 128, BOGUS, BOGUS, 16, BOGUS, BOGUS, ctypes.byref(n), None) == INVALID
    assert g(BOGUS, BOGUS, 4, 128, BOGUS, BOGUS, 16, BOGUS, BOGUS, None, None) == INVALID
    # K = 7168 is cut into slices whose partial sums need a workspace; the
    # shape is checked to need one before a too-small one is passed (with
    # bogus pointers a call must never get past validation)
    need = ctypes.c_size_t(0)
    assert g(None, None, 4, 7168, None, None, 16, None, None, ctypes.byref(need), None) == OK
    assert need.value > 8
    small = ctypes.c_size_t(8)
    assert g(BOGUS, BOGUS, 4, 7168, BOGUS, BOGUS, 16, BOGUS, BOGUS, ctypes.byref(small), None) == WORKSPACE


def test_align_rejects_bad_arguments(L):
    n = ctypes.c_size_t(1 << 40)
    a = L.w4a8_moe_align
    args = lambda T=4, k=2, E=4, bm=16, ids=BOGUS, be=BOGUS, br=BOGUS: a(
        ids, T, k, 0, E, bm, BOGUS, BOGUS, BOGUS, BOGUS, be, br, BOGUS, BOGUS, ctypes.byref(n), None)
    assert args(k=0) == INVALID
    assert args(k=33) == UNSUPPORTED
    assert args(E=0) == INVALID
    assert args(E=1025) == UNSUPPORTED
    assert args(bm=0) == INVALID
    assert args(ids=None) == INVALID
    assert args(be=None) == INVALID  # block_expert and block_row must both be given or both null


def test_prepack_rejects_bad_arguments(L):
    p = L.w4a8_prepack_weights
    other = ctypes.c_void_p(0x2000)
    args = lambda E=2, N=32, K=256, w=BOGUS, s=BOGUS, wp=other, sp=other: p(w, s, E, N, K, wp, sp, None)
    assert args(E=0) == INVALID
    assert args(N=0) == INVALID
    assert args(K=-128) == INVALID
    assert args(w=None) == INVALID
    assert args(sp=None) == INVALID
    assert args(N=24) == UNSUPPORTED        # N % 16
    assert args(K=192) == UNSUPPORTED       # K % 128
    assert args(w=MISALIGNED) == UNSUPPORTED
    assert args(sp=MISALIGNED) == UNSUPPORTED
    assert args(wp=BOGUS) == INVALID        # in place


def test_prepacked_scale_count(L):
    c = L.w4a8_prepacked_scale_count
    # groups are padded to a multiple of 4 per row
    assert c(1, 16, 128) == 16 * 4
    assert c(3, 32, 512) == 3 * 32 * 4
    assert c(2, 48, 640) == 2 * 48 * 8      # 5 groups -> 8
    assert c(256, 4096, 7168) == 256 * 4096 * 56
    assert c(0, 16, 128) == -1
    assert c(1, 16, 100) == -1


def test_fused_moe_prepacked_rejects_bad_arguments(L):
    n = ctypes.c_size_t(1 << 40)
    f = lambda H=256, I=128, w13=BOGUS, nbytes=n: L.w4a8_fused_moe_prepacked(
        BOGUS, 4, H, BOGUS, BOGUS, 2, 0, 4, I, w13, BOGUS, BOGUS, BOGUS, BOGUS, BOGUS,
        ctypes.byref(nbytes), None)
    assert f(H=200) == UNSUPPORTED
    assert f(I=100) == UNSUPPORTED
    assert f(w13=None) == INVALID
    assert f(nbytes=ctypes.c_size_t(16)) == WORKSPACE


def test_prepack_fp4_rejects_bad_arguments(L):
    p = L.w4a8_prepack_weights_fp4
    other = ctypes.c_void_p(0x2000)
    args = lambda E=2, N=32, K=256, role=0, w=BOGUS, s=BOGUS, wp=other, sp=other: p(
        w, s, E, N, K, role, wp, sp, None)
    assert args(role=2) == INVALID
    assert args(role=-1) == INVALID
    assert args(E=0) == INVALID
    assert args(s=None) == INVALID
    assert args(N=40) == UNSUPPORTED
    assert args(K=160) == UNSUPPORTED
    assert args(s=ctypes.c_void_p(0x1002)) == UNSUPPORTED   # scales need 4-byte alignment
    assert args(wp=MISALIGNED) == UNSUPPORTED
    assert args(sp=BOGUS) == INVALID                        # in place


def test_fused_moe_fp4_rejects_bad_arguments(L):
    n = ctypes.c_size_t(1 << 40)
    f = lambda H=256, I=128, w13=BOGUS, nbytes=n: L.w4a8_fused_moe_fp4_prepacked(
        BOGUS, 4, H, BOGUS, BOGUS, 2, 0, 4, I, w13, BOGUS, BOGUS, BOGUS, BOGUS, BOGUS,
        ctypes.byref(nbytes), None)
    assert f(H=200) == UNSUPPORTED
    assert f(w13=None) == INVALID
    assert f(nbytes=ctypes.c_size_t(16)) == WORKSPACE


def test_prepack_bf16_scales_rejects_bad_arguments(L):
    p = L.w4a8_prepack_weights_bf16_scales
    other = ctypes.c_void_p(0x2000)
    args = lambda E=2, N=32, K=256, w=BOGUS, s=BOGUS, wp=other, sp=other: p(w, s, E, N, K, wp, sp, None)
    assert args(E=0) == INVALID
    assert args(s=None) == INVALID
    assert args(N=24) == UNSUPPORTED
    assert args(s=ctypes.c_void_p(0x1001)) == UNSUPPORTED   # bf16 needs 2-byte alignment
    assert args(sp=MISALIGNED) == UNSUPPORTED
    assert args(wp=BOGUS) == INVALID                         # in place


def test_fused_moe_static_rejects_bad_arguments(L):
    n = ctypes.c_size_t(1 << 40)
    f = lambda H=256, a1=None, a2=None, nbytes=n: L.w4a8_fused_moe_prepacked_static(
        BOGUS, 4, H, BOGUS, BOGUS, 2, 0, 4, 128, BOGUS, BOGUS, BOGUS, BOGUS, a1, a2, BOGUS, BOGUS,
        ctypes.byref(nbytes), None)
    assert f(H=200) == UNSUPPORTED
    assert f(a1=ctypes.c_void_p(0x1002)) == UNSUPPORTED   # scale pointers need 4-byte alignment
    assert f(nbytes=ctypes.c_size_t(16)) == WORKSPACE


def test_fused_moe_recipe_rejects_bad_arguments(L):
    n = ctypes.c_size_t(1 << 40)
    f = lambda fmt=1, group=64, nbytes=n: L.w4a8_fused_moe_recipe(
        BOGUS, 4, 256, BOGUS, BOGUS, 2, 0, 4, 128, fmt, BOGUS, BOGUS, BOGUS, BOGUS, group, BOGUS,
        BOGUS, ctypes.byref(nbytes), None)
    assert f(fmt=0) == INVALID       # canonical weights are not a recipe format
    assert f(fmt=3) == INVALID
    assert f(group=48) == INVALID
    assert f(group=16) == INVALID
    assert f(nbytes=ctypes.c_size_t(16)) == WORKSPACE
    assert f(group=32, nbytes=ctypes.c_size_t(16)) == WORKSPACE


@pytest.mark.parametrize("T,topk,E,want,two", [
    (64, 8, 32, 16, False),     # decode share: 16 pairs per local expert if all were local
    (1, 8, 256, 16, False),
    (128, 8, 32, 16, True),     # 32: per-expert 16 / 32-row blocks, chosen on the device
    (256, 8, 32, 16, True),
    (1023, 8, 32, 16, True),    # 8184 pairs: one short of 256 per expert
    (1024, 8, 32, 160, False),  # 8192 pairs: the block-tiled kernel's 160-row m-blocks
    (4096, 8, 32, 160, False),
])
def test_block_height_rule(L, T, topk, E, want, two):
    """The m-block height(s) the fused call picks from the pairs per local
    expert (host-side, from the shapes alone), and a layout consistent with
    it: the first list's blocks of `want` rows, and with two lists a second
    list of 32-row blocks behind the other buffers."""
    lay = w4.fused_moe_workspace_layout(T, 7168, topk, E, 2048)
    assert lay["block_m"] == want
    assert lay["two_lists"] == two
    # between the two host rules the path is chosen on the device (a third,
    # 160-row list and the path flag behind the others)
    assert lay["device_path"] == two
    F = T * topk
    keys = list(w4.LAYOUT_KEYS) if two else list(w4.LAYOUT_KEYS)[:12]
    offs = [lay[k] for k in keys]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    # block lists hold at most ceil(F / block_m) + E entries
    nb_max = (F + want - 1) // want + E
    assert lay["block_row"] - lay["block_expert"] >= 4 * nb_max
    if two:
        assert lay["block_row2"] - lay["block_expert2"] >= 4 * ((F + 31) // 32 + E)
        assert lay["num_blocks3"] - lay["block_row3"] >= 4 * ((F + 159) // 160 + E)
    else:
        assert lay["block_expert2"] == lay["block_row2"] == lay["num_blocks2"] == 0
        assert lay["block_row3"] == lay["num_blocks3"] == lay["path"] == 0


def _bounded(L, T=4, H=256, k=2, E=4, I=128, fmt=1, bound=8, pairs=BOGUS, ws=BOGUS, nbytes=None):
    n = ctypes.c_size_t(1 << 62) if nbytes is None else nbytes
    return L.w4a8_fused_moe_bounded(BOGUS, T, H, BOGUS, BOGUS, k, 0, E, I, fmt, BOGUS, BOGUS, BOGUS,
                                    BOGUS, bound, pairs, BOGUS, ws, ctypes.byref(n), None)


def test_fused_moe_bounded_rejects_bad_arguments(L):
    assert _bounded(L, fmt=3) == INVALID
    assert _bounded(L, fmt=-1) == INVALID
    assert _bounded(L, bound=0) == INVALID
    assert _bounded(L, pairs=None) == INVALID          # the pair count has nowhere to go
    assert _bounded(L, pairs=ctypes.c_void_p(0x1004)) == UNSUPPORTED  # int32[2] needs 8-byte alignment
    assert _bounded(L, nbytes=ctypes.c_size_t(16)) == WORKSPACE
    # the query needs no pair-count pointer
    n = ctypes.c_size_t(0)
    assert _bounded(L, pairs=None, ws=None, nbytes=n) == OK and n.value > 0


def test_fused_moe_bounded_workspace_scales_with_the_bound(L):
    """The per-pair buffers follow the bound: the EP8 share of a 32768-token
    prefill (32 of 256 experts, top-8: ~33000 local pairs of 262144) needs
    about an eighth of the unbounded workspace; a bound at or above T*topk
    sizes it like the unbounded call."""
    T, H, k, E, I = 32768, 7168, 8, 32, 2048
    full = w4.fused_moe_workspace_bytes(T, H, k, E, I)
    assert full > 8.4e9  # 8.4 GB, 7.5 GB of it the fp32 down output
    b = w4.fused_moe_bounded_workspace_bytes(T, H, k, E, I, 40000)
    assert b < full / 5
    # the fp32 down output dominates: about bound * H * 4 bytes plus T*H fp8 codes
    assert 40000 * H * 4 < b < 40000 * (H * 4 + I * 2) + T * (H + 8 * H // 128) + (64 << 20)
    for fmt in (0, 1, 2):
        assert w4.fused_moe_bounded_workspace_bytes(T, H, k, E, I, T * k, fmt) == full
        assert w4.fused_moe_bounded_workspace_bytes(T, H, k, E, I, 1 << 40, fmt) == full
    small = w4.fused_moe_bounded_workspace_bytes(64, H, k, E, I, 64)
    assert small < w4.fused_moe_workspace_bytes(64, H, k, E, I)


def test_fused_moe_bounded_range_check_uses_the_bound(L):
    """The down GEMM's activation rows are bound*I bytes: T*topk*I >= 2^32 is
    accepted under a bound that keeps it below, rejected under one that does
    not (validation returns before any launch: the query path)."""
    n = ctypes.c_size_t(0)
    assert _bounded(L, T=262144, H=128, k=8, E=32, I=2048, bound=100000, ws=None, nbytes=n) == OK
    assert _bounded(L, T=262144, H=128, k=8, E=32, I=2048, bound=1 << 21, ws=None,
                    nbytes=ctypes.c_size_t(0)) == UNSUPPORTED


def _persistent(L, T=4, H=256, k=2, E=4, I=128, fmt=1, ws=BOGUS, nbytes=None, out=BOGUS):
    n = ctypes.c_size_t(1 << 62) if nbytes is None else nbytes
    return L.w4a8_fused_moe_persistent(BOGUS, T, H, BOGUS, BOGUS, k, 0, E, I, fmt, BOGUS, BOGUS,
                                       BOGUS, BOGUS, out, ws, ctypes.byref(n), None)


def test_fused_moe_persistent_rejects_bad_arguments(L):
    assert _persistent(L, fmt=3) == INVALID
    assert _persistent(L, fmt=-1) == INVALID
    assert _persistent(L, H=200) == UNSUPPORTED
    assert _persistent(L, k=0) == INVALID
    assert _persistent(L, out=None) == INVALID
    assert _persistent(L, out=MISALIGNED) == UNSUPPORTED
    assert _persistent(L, nbytes=ctypes.c_size_t(16)) == WORKSPACE
    assert _persistent(L, T=1, H=(1 << 24) + 128, ws=None, nbytes=ctypes.c_size_t(0)) == UNSUPPORTED


def test_fused_moe_persistent_workspace(L):
    """The single-launch call always runs the block-tiled kernels (160-row
    m-blocks): its workspace is the block-tiled plan's plus the grid-barrier
    counter, so at a shape the multi-launch call also runs tiled (T*topk/E_l
    >= 256) it is that call's size plus one 256-byte slot, and at decode it
    differs from the skinny plan's only in the block lists."""
    H, k, E, I = 7168, 8, 32, 2048
    for fmt in (0, 1, 2):
        n = ctypes.c_size_t(0)
        assert _persistent(L, T=4096, H=H, k=k, E=E, I=I, fmt=fmt, ws=None, nbytes=n) == OK
        assert n.value == w4.fused_moe_workspace_bytes(4096, H, k, E, I) + 256
    n = ctypes.c_size_t(0)
    assert _persistent(L, T=64, H=H, k=k, E=E, I=I, ws=None, nbytes=n) == OK
    assert abs(n.value - w4.fused_moe_workspace_bytes(64, H, k, E, I)) < (1 << 16)
