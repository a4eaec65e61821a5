"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars:
  * quantisation codes and scales, routing permutation: bit-exact;
  * bf16 outputs of the GEMM and the fused MoE: relative Frobenius error
    <= 1e-3 and max |diff| <= 2e-2 * max |ref| against the oracle's fp64 result
    rounded to bf16; rows the oracle gives exactly +0 (no local pair) must be
    exactly +0.
Full-size workloads are checked on sampled tokens: every output row depends
only on its own token (plus the weights), so the oracle run on the sampled
tokens alone gives exactly those rows.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from w4a8_moe_grouped_amd import lib as w4
from w4a8_moe_grouped_amd import synth

pytestmark = pytest.mark.gpu

REL_FRO = 1e-3
MAX_REL = 2e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    w4.load()
    return torch.device("cuda:0")


def dput(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_dev(bits, dev):
    return dput(np.ascontiguousarray(bits).view(np.int16), dev).view(torch.bfloat16)


def bf16_host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bf16_close(got_bits, ref_bits, what=""):
    g = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    r = synth.bf16_bits_to_f32(ref_bits).astype(np.float64)
    assert np.all(np.isfinite(g)), what
    zero_rows = np.all(r == 0, axis=-1)
    if np.any(zero_rows):
        assert np.all(got_bits[zero_rows] == 0), "%s: rows without local pairs must be +0" % what
    nr = np.linalg.norm(r)
    if nr == 0:
        assert np.all(got_bits == 0), what
        return
    fro = np.linalg.norm(g - r) / nr
    mx = np.max(np.abs(g - r)) / np.max(np.abs(r))
    print("%s: rel_fro=%.3e max_rel=%.3e" % (what, fro, mx))
    assert fro <= REL_FRO and mx <= MAX_REL, (what, fro, mx)


_cache = {}


def moe_inputs(name):
    if name not in _cache:
        cfg = synth.CONFIGS[name]
        _cache[name] = (cfg, synth.gen_moe(cfg))
    return _cache[name]


# ---------------------------------------------------------------------------
# activation quantisation: bit-exact
# ---------------------------------------------------------------------------

def check_quant(x_bits, dev, ldx_pad=0):
    M, K = x_bits.shape
    if ldx_pad:
        buf = np.zeros((M, K + ldx_pad), np.uint16)
        buf[:, :K] = x_bits
        xd = bf16_dev(buf, dev)[:, :K]
    else:
        xd = bf16_dev(x_bits, dev)
    q, s = w4.quantize_act(xd)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_bf16(x_bits)
    gq, gs = q.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(gq, rq), "codes differ at %s" % (np.argwhere(gq != rq)[:5],)
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "decode", "skew_perm"])
def test_quant_bit_exact_moe_hidden(dev, name):
    cfg = synth.CONFIGS[name]
    check_quant(synth.gen_hidden(cfg), dev)


def test_quant_bit_exact_dense_with_outliers(dev):
    x, _, _ = synth.gen_dense(synth.CONFIGS["dense"])
    check_quant(x, dev)
    check_quant(x[:37], dev, ldx_pad=64)  # ragged M, row stride > K


def test_quant_edge_rows(dev):
    rng = np.random.default_rng(0)
    rows = []
    rows.append(np.zeros(256, np.float32))                       # all zero -> clamped amax
    r = np.zeros(256, np.float32); r[3] = -2.5; rows.append(r)   # single nonzero
    rows.append(np.full(256, 3e38, np.float32))                  # huge
    rows.append(np.full(256, 1e-38, np.float32))                 # tiny, below the clamp
    rows.append(rng.normal(size=256).astype(np.float32) * 1e-12)
    r = rng.normal(size=256).astype(np.float32); r[::7] = 0; rows.append(r)
    rows.append(np.linspace(-448, 448, 256).astype(np.float32))
    x = synth.to_bf16_bits(np.stack(rows))
    x[4, 10] = 0x0001   # bf16 subnormal
    x[5, 11] = 0x8000   # -0
    check_quant(x, dev)
    check_quant(x[:1], dev)


def test_quant_every_bf16_amax_and_element(dev):
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)  # every positive finite bf16
    rng = np.random.default_rng(1)
    x = np.zeros((bits.size, 128), np.uint16)
    x[:, 5] = bits
    x[:, 77] = bits | 0x8000
    # the other entries: every bf16 value again, shuffled, scaled below the row's amax
    other = rng.permutation(bits)
    small = np.minimum(synth.bf16_bits_to_f32(other), synth.bf16_bits_to_f32(bits))
    x[:, 9] = synth.to_bf16_bits(small)
    x[:, 100] = synth.to_bf16_bits(-small * np.float32(0.7))
    check_quant(x, dev)


# ---------------------------------------------------------------------------
# routing permutation: bit-exact
# ---------------------------------------------------------------------------

def check_align(ids, eb, E, bm, dev):
    g = w4.moe_align(dput(ids.astype(np.int32), dev), eb, E, bm)
    torch.cuda.synchronize()
    r = oracle.moe_align(ids, eb, E, bm)
    P = int(r["offsets"][-1])
    nb = int(g["num_blocks"].item())
    assert nb == r["num_blocks"]
    assert np.array_equal(g["counts"].cpu().numpy(), r["counts"])
    assert np.array_equal(g["offsets"].cpu().numpy(), r["offsets"])
    assert np.array_equal(g["sorted_pair_ids"].cpu().numpy()[:P], r["sorted_pair_ids"])
    F = ids.size
    assert np.array_equal(g["src2dst"].cpu().numpy()[:F], r["src2dst"])
    assert np.array_equal(g["block_expert"].cpu().numpy()[:nb], r["block_expert"])
    assert np.array_equal(g["block_row"].cpu().numpy()[:nb], r["block_row"])


@pytest.mark.parametrize("name,bm", [("tiny", 16), ("decode", 16), ("prefill", 64),
                                     ("prefill_ep8", 128), ("skew_perm", 64), ("skew_id", 32)])
def test_align_bit_exact_configs(dev, name, bm):
    cfg = synth.CONFIGS[name]
    ids, _ = synth.gen_routing(cfg)
    check_align(ids, cfg.expert_begin, cfg.E_local, bm, dev)


@pytest.mark.parametrize("T,k,eb,E,bm,seed", [
    (1, 1, 0, 1, 1, 0), (1, 8, 0, 32, 16, 1), (3, 32, 5, 7, 3, 2), (600, 8, 40, 32, 16, 3),
    (5000, 6, 0, 1024, 64, 4), (4097, 1, 0, 3, 100, 5), (20000, 8, 224, 32, 64, 6),
    (512, 8, 0, 1024, 16, 7), (256, 8, 0, 32, 64, 8), (1024, 4, 2, 2, 160, 9)])
def test_align_bit_exact_random(dev, T, k, eb, E, bm, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, eb + E + 9, size=(T, k)).astype(np.int32)
    ids[rng.uniform(size=(T, k)) < 0.1] = -1
    check_align(ids, eb, E, bm, dev)


def test_align_all_non_local_and_one_hot(dev):
    ids = np.full((300, 4), 77, np.int32)
    check_align(ids, 0, 8, 16, dev)             # P = 0
    ids = np.full((300, 4), 3, np.int32)
    check_align(ids, 0, 8, 16, dev)             # everything on one expert


# ---------------------------------------------------------------------------
# dense GEMM: tolerance
# ---------------------------------------------------------------------------

def check_gemm(x_bits, w, sw, dev, what):
    xd = bf16_dev(x_bits, dev)
    q, s = w4.quantize_act(xd)
    out = w4.gemm(q, s, dput(w, dev), dput(sw, dev))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_bf16(x_bits)
    ref = oracle.gemm_bf16(rq, rs, w, sw)
    assert_bf16_close(bf16_host(out), ref, what)


def test_gemm_dense_config(dev):
    x, w, sw = synth.gen_dense(synth.CONFIGS["dense"])
    check_gemm(x, w, sw, dev, "dense M=128 K=7168 N=2048")


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (5, 384, 40), (33, 256, 300), (70, 1024, 513),
                                   (17, 7168, 256), (64, 2048, 7168),
                                   # few tiles: K split over workgroups, partials reduced in order
                                   (1, 7168, 2048), (4, 7168, 256), (5, 7168, 256), (16, 2048, 512),
                                   # 16-row blocks, K % 1024 == 0 and enough tiles to run unsplit:
                                   # the whole-K rows staged in LDS
                                   (3, 1024, 65536)])
def test_gemm_ragged_shapes(dev, M, K, N):
    rng = np.random.default_rng(M * 7 + N)
    x = synth.to_bf16_bits(rng.normal(size=(M, K)).astype(np.float32))
    w = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sw = rng.uniform(0.002, 0.02, size=(N, K // 128)).astype(np.float32)
    check_gemm(x, w, sw, dev, "gemm %dx%dx%d" % (M, K, N))


# ---------------------------------------------------------------------------
# fused MoE: tolerance
# ---------------------------------------------------------------------------

def run_fused(d, cfg, dev):
    out = w4.fused_moe(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev),
                       dput(d["topk_weights"], dev), cfg.expert_begin, cfg.E_local,
                       dput(d["w13"], dev), dput(d["s13"], dev), dput(d["w2"], dev),
                       dput(d["s2"], dev))
    torch.cuda.synchronize()
    return bf16_host(out)


def oracle_rows(d, cfg, rows):
    return oracle.fused_moe(d["hidden"][rows], d["topk_ids"][rows], d["topk_weights"][rows],
                            cfg.expert_begin, cfg.E_local, d["w13"], d["s13"], d["w2"], d["s2"])


ORACLE_THREADS = 16  # the host's share of the box


def oracle_rows_parallel(d, cfg, rows, fn=None, threads=ORACLE_THREADS):
    """The oracle on the given tokens, split over threads (every output row
    depends only on its own token, so the slices' rows equal one call's)."""
    import concurrent.futures
    fn = fn or oracle.fused_moe
    rows = np.asarray(rows)
    parts = [p for p in np.array_split(rows, min(threads, rows.size)) if p.size]

    def run(r):
        return fn(d["hidden"][r], d["topk_ids"][r], d["topk_weights"][r], cfg.expert_begin,
                  cfg.E_local, d["w13"], d["s13"], d["w2"], d["s2"])
    with concurrent.futures.ThreadPoolExecutor(len(parts)) as ex:
        outs = list(ex.map(run, parts))
    return np.concatenate(outs, axis=0)


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_fused_moe_full(dev, name):
    cfg, d = moe_inputs(name)
    got = run_fused(d, cfg, dev)
    ref = oracle_rows(d, cfg, np.arange(cfg.T))
    assert_bf16_close(got, ref, name)


@pytest.mark.parametrize("name,nsample", [("skew_perm", 40), ("skew_id", 24), ("prefill", 24),
                                          ("prefill_ep8", 16)])
def test_fused_moe_sampled_tokens(dev, name, nsample):
    cfg, d = moe_inputs(name)
    got = run_fused(d, cfg, dev)
    rng = np.random.default_rng(123)
    rows = np.sort(rng.choice(cfg.T, size=nsample, replace=False))
    rows[0], rows[-1] = 0, cfg.T - 1
    ref = oracle_rows(d, cfg, rows)
    assert_bf16_close(got[rows], ref, "%s (%d sampled tokens)" % (name, nsample))
    # rows with no local pair must be exactly zero everywhere
    ids = d["topk_ids"]
    none_local = ~np.any((ids >= cfg.expert_begin) & (ids < cfg.expert_begin + cfg.E_local), axis=1)
    assert np.all(got[none_local] == 0)


# Per-expert block heights at the model's dimensions (H=7168, I=2048: 56 and
# 16 K-groups): Zipf routing with rank = expert id puts 1..60 pairs on the
# local experts, so both m-block lists (16 rows for experts with at most 16
# pairs, 32 rows -- activation rows through LDS once per workgroup -- for the
# others) hold blocks; one token of every local expert is compared.
def test_fused_moe_two_block_lists_full_dims(dev):
    cfg, d = synth.random_moe(128, 7168, 2048, 256, 8, 0, 32, seed=71, routing="zipf_id")
    lay = w4.fused_moe_workspace_layout(cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I)
    assert lay["block_m"] == 16 and lay["two_lists"], lay
    counts = np.bincount(d["topk_ids"].ravel(), minlength=cfg.E_total)[:cfg.E_local]
    assert np.any((counts > 0) & (counts <= 16)) and np.any(counts > 16), counts
    got = run_fused(d, cfg, dev)
    rows = set()
    for e in range(cfg.E_local):  # the first and the last token of every local expert
        toks = np.nonzero(np.any(d["topk_ids"] == e, axis=1))[0]
        if toks.size:
            rows.update((int(toks[0]), int(toks[-1])))
    rows = np.array(sorted(rows))
    ref = oracle_rows_parallel(d, cfg, rows)
    assert_bf16_close(got[rows], ref, "T=128 per-expert 16 / 32-row blocks (%d tokens)" % rows.size)


@pytest.mark.parametrize("case", ["one_expert_many_rows", "single_token", "k1_e1",
                                  "non_local_mix", "topk32", "small_dims", "all_non_local",
                                  "two_slices", "g3_16row", "g3_32row", "staged_and_not_16row"])
def test_fused_moe_edge_cases(dev, case):
    if case == "one_expert_many_rows":   # every pair on expert 2: many full blocks + a partial one
        cfg, d = synth.random_moe(150, 256, 256, 8, 2, 0, 8, seed=21)
        d["topk_ids"][:, 0] = 2
    elif case == "single_token":
        cfg, d = synth.random_moe(1, 7168, 2048, 256, 8, 0, 256, seed=22)
    elif case == "k1_e1":
        cfg, d = synth.random_moe(40, 384, 128, 1, 1, 0, 1, seed=23)
        d["topk_weights"][:] = 1.0
    elif case == "non_local_mix":
        cfg, d = synth.random_moe(64, 256, 128, 16, 4, 8, 4, seed=24)
        d["topk_ids"][:10] = -1
    elif case == "topk32":
        cfg, d = synth.random_moe(9, 256, 128, 64, 32, 0, 64, seed=25)
    elif case == "two_slices":      # ~30 rows per expert: 32-row blocks with both 16-row slices
        cfg, d = synth.random_moe(120, 256, 128, 4, 1, 0, 4, seed=28)
    elif case == "g3_16row":        # 16-row blocks, down K = 384: 3 groups, ring of 4, shared rows
        cfg, d = synth.random_moe(64, 256, 384, 64, 8, 0, 32, seed=29)
    elif case == "g3_32row":        # 32-row blocks, K = 384 both GEMMs: 3 groups, ring of 2, shared rows
        cfg, d = synth.random_moe(96, 384, 384, 32, 4, 8, 16, seed=30)
    elif case == "staged_and_not_16row":  # ~16 rows per expert, down K = 2048: blocks with up to
        # 11 rows read a whole-K copy from LDS, fuller ones the per-group path
        cfg, d = synth.random_moe(128, 256, 2048, 64, 8, 0, 64, seed=37)
    elif case == "all_non_local":   # no m-block at all: the output is +0 everywhere
        cfg, d = synth.random_moe(48, 256, 128, 8, 2, 4, 4, seed=27)
        d["topk_ids"][:] = d["topk_ids"] % 4
    else:
        cfg, d = synth.random_moe(33, 128, 128, 4, 3, 1, 2, seed=26)
    got = run_fused(d, cfg, dev)
    ref = oracle_rows(d, cfg, np.arange(cfg.T))
    assert_bf16_close(got, ref, case)


# Block-tiled path (many rows per local expert): 160-row m-blocks, ragged
# last blocks, a partial 256-wide weight block, fewer K-groups than pipeline
# stages, an expert with no rows next to one with many.
def tile_case(case):
    if case == "tile_small":        # ~128 rows per expert: one m-block, partial second half
        return synth.random_moe(512, 256, 256, 8, 2, 0, 4, seed=31)
    if case == "tile_two_blocks":   # ~170 rows per expert: full + nearly empty m-blocks
        return synth.random_moe(680, 256, 256, 8, 2, 0, 4, seed=34)
    if case == "tile_ragged":       # H = 384: down weight blocks 256 + 128; 3 and 1 K-groups
        return synth.random_moe(700, 384, 128, 5, 2, 1, 3, seed=32)
    if case == "tile_boundaries":   # 80 / 81 / 160 / 161 rows: idle half, one-row half, full, one-row block
        cfg, d = synth.random_moe(512, 256, 256, 8, 2, 0, 4, seed=35)
        rows = np.concatenate([np.full(n, e) for e, n in enumerate((80, 81, 160, 161))])
        rng = np.random.default_rng(35)
        flat = np.concatenate([rows, rng.integers(4, 8, size=cfg.T * cfg.topk - rows.size)])
        d["topk_ids"][:] = rng.permutation(flat).reshape(cfg.T, cfg.topk).astype(np.int32)
        return cfg, d
    cfg, d = synth.random_moe(300, 256, 256, 4, 2, 0, 2, seed=33)
    d["topk_ids"][:] = 1            # every pair on local expert 1, expert 0 empty: 4 m-blocks
    return cfg, d


@pytest.mark.parametrize("case", ["tile_small", "tile_two_blocks", "tile_ragged", "tile_one_expert",
                                  "tile_boundaries"])
def test_fused_moe_tile_path(dev, case):
    cfg, d = tile_case(case)
    lay = w4.fused_moe_workspace_layout(cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I)
    assert lay["block_m"] == 160, "expected the block-tiled path"
    got = run_fused(d, cfg, dev)
    ref = oracle_rows(d, cfg, np.arange(cfg.T))
    assert_bf16_close(got, ref, case)


def test_fused_moe_repeatable_and_workspace_reuse(dev):
    cfg, d = moe_inputs("tiny")
    a = run_fused(d, cfg, dev)
    b = run_fused(d, cfg, dev)
    assert np.array_equal(a, b)


# The output and the workspace start as all-ones bytes (bf16 NaN, counters at
# -1): every output element, including the +0 rows of tokens without a local
# expert, must be written by the call, and the summation counters of the
# fused combine must be cleared by the call itself.  Two calls in a row on the
# same buffers, the second with other routing and fewer tokens.
@pytest.mark.parametrize("case", ["skinny16", "lists_small", "lists_large", "tile", "chunked_tile",
                                  "chunked_lists"])
def test_fused_moe_poisoned_buffers(dev, case):
    # skinny16: one list of 16-row blocks; lists_small / lists_large: per-expert
    # 16 / 32-row blocks with ~12 / ~40 pairs per local expert; tile: 160 rows;
    # chunked_tile / chunked_lists: more than 4096 pairs (the chunked align)
    # with top-6 (tokens straddle the 1024-pair chunks) and 1/8 of the
    # experts local (block-tiled / device-chosen path)
    shapes = {"skinny16": (64, 256, 128, 64, 8, 0, 32),
              "lists_small": (96, 256, 128, 32, 4, 8, 16),
              "lists_large": (160, 256, 128, 16, 4, 0, 8),
              "tile": (512, 256, 256, 8, 2, 0, 4),
              "chunked_tile": (1000, 256, 128, 64, 6, 8, 8),
              "chunked_lists": (900, 256, 128, 256, 6, 0, 32)}[case]
    T, H, I, E, k, eb, El = shapes
    cfg1, d1 = synth.random_moe(T, H, I, E, k, eb, El, seed=61)
    cfg2, d2 = synth.random_moe(T - 7, H, I, E, k, eb, El, seed=62)
    d2["topk_ids"][:5] = -1  # tokens with no expert at all
    need = w4.fused_moe_workspace_bytes(T, H, k, El, I)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    out = torch.full((T, H), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
    lay = w4.fused_moe_workspace_layout(T, H, k, El, I)
    assert lay["block_m"] == {"skinny16": 16, "lists_small": 16, "lists_large": 16, "tile": 160,
                              "chunked_tile": 160, "chunked_lists": 16}[case]
    assert lay["two_lists"] == (case in ("lists_small", "lists_large", "chunked_lists"))
    w = [tuple(dput(d[n], dev) for n in ("w13", "s13", "w2", "s2")) for d in (d1, d2)]
    for cfg, d, wt in ((cfg1, d1, w[0]), (cfg2, d2, w[1])):
        o = out[:cfg.T]
        w4.fused_moe(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev), dput(d["topk_weights"], dev),
                     cfg.expert_begin, cfg.E_local, *wt, out=o, workspace=ws)
        torch.cuda.synchronize()
        got = bf16_host(o)
        ref = oracle_rows(d, cfg, np.arange(cfg.T))
        assert not np.any(np.isnan(got)), case
        ids = d["topk_ids"]
        none_local = ~np.any((ids >= cfg.expert_begin) & (ids < cfg.expert_begin + cfg.E_local), axis=1)
        assert np.all(got[none_local] == 0), case
        assert_bf16_close(got, ref, case)


# Many local experts (beyond the align's 256 threads per pass): 600 local
# experts with ~40 pairs each take the device-chosen path (the align sums the
# cost of every expert's tiles over several passes), 1024 (the largest E_l)
# the two skinny lists; every token is compared.
@pytest.mark.parametrize("E", [600, 1024])
def test_fused_moe_many_local_experts(dev, E):
    cfg, d = synth.random_moe(3000, 256, 128, E, 8, 0, E, seed=121)
    lay = w4.fused_moe_workspace_layout(cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I)
    assert lay["two_lists"] and lay["device_path"] == (E == 600), lay
    need = w4.fused_moe_workspace_bytes(cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    out = torch.full((cfg.T, cfg.H), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
    w4.fused_moe(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev), dput(d["topk_weights"], dev),
                 cfg.expert_begin, cfg.E_local, dput(d["w13"], dev), dput(d["s13"], dev),
                 dput(d["w2"], dev), dput(d["s2"], dev), out=out, workspace=ws)
    torch.cuda.synchronize()
    got = bf16_host(out)
    ref = oracle_rows_parallel(d, cfg, np.arange(cfg.T))
    assert_bf16_close(got, ref, "E_l=%d" % E)
