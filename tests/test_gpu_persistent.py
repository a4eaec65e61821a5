"""The fused forward with everything after the align in one launch
(w4a8_fused_moe_persistent; DeepGEMM PR #53, "Changes": one persistent kernel
runs L1 GEMM -> SwiGLU -> FP8 requant -> L2 GEMM -> combine), through the C ABI.

* Its arithmetic is the block-tiled path's, so where the multi-launch exports
  run the block-tiled kernels (T*topk/E_l >= 256: the 4096-token prefill and
  the EP8 share of a 32768-token one) the output is bit-identical to theirs,
  for every weight format; a few rows are also held to the oracle directly.
* At every other size it runs the block-tiled kernels too (160-row m-blocks
  for a handful of rows, most workgroups idle in the GEMM phases), held to the
  oracle's bar on all rows: the tiny config, decode, ragged shapes, tokens
  with no expert at all and with no local expert.
* The grid-barrier counter lives in the workspace and the align clears it:
  a workspace filled with 0xFF bytes, and calls of different shapes one after
  another on the same workspace, give the same results.
"""
import numpy as np
import pytest
import torch

from w4a8_moe_grouped_amd import lib as w4
from w4a8_moe_grouped_amd import synth

from test_gpu_bounded import weights
from test_gpu_parity import (assert_bf16_close, bf16_dev, bf16_host, dput, moe_inputs,
                             oracle_rows_parallel)

pytestmark = pytest.mark.gpu

FORMATS = [w4.WEIGHTS_INT4, w4.WEIGHTS_INT4_PACKED, w4.WEIGHTS_FP4_PACKED]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    w4.load()
    return torch.device("cuda:0")


def persistent(d, cfg, dev, fmt, wts, out=None, workspace=None):
    o = w4.fused_moe_persistent(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev),
                                dput(d["topk_weights"], dev), cfg.expert_begin, cfg.E_local, cfg.I,
                                wts, fmt, out=out, workspace=workspace)
    torch.cuda.synchronize()
    return bf16_host(o)


def multi_launch(d, cfg, dev, fmt, wts):
    """The same forward through the multi-launch export of the same format
    (bounded by T*topk, which sizes and chooses exactly as the unbounded
    call does)."""
    out, _ = w4.fused_moe_bounded(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev),
                                  dput(d["topk_weights"], dev), cfg.expert_begin, cfg.E_local, cfg.I,
                                  wts, fmt, cfg.T * cfg.topk)
    torch.cuda.synchronize()
    return bf16_host(out)


def oracle_fn(fmt):
    import oracle
    return oracle.fused_moe_fp4 if fmt == w4.WEIGHTS_FP4_PACKED else oracle.fused_moe


_fp4_weights = {}


def with_fp4_weights(cfg, d):
    """The same routing and activations with fp4 weights of the same shapes."""
    key = (cfg.E_local, cfg.H, cfg.I, cfg.seed)
    if key not in _fp4_weights:
        _fp4_weights[key] = synth.gen_expert_weights_fp4(cfg)
    d = dict(d)
    d["w13"], d["s13"], d["w2"], d["s2"] = _fp4_weights[key]
    return d


def no_local_rows(cfg, d):
    ids = d["topk_ids"]
    return ~np.any((ids >= cfg.expert_begin) & (ids < cfg.expert_begin + cfg.E_local), axis=1)


@pytest.mark.parametrize("name", ["prefill", "prefill_ep8"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_persistent_bit_identical_to_tiled_launches(dev, name, fmt):
    cfg, d = moe_inputs(name)
    if fmt == w4.WEIGHTS_FP4_PACKED:
        d = with_fp4_weights(cfg, d)
    lay = w4.fused_moe_workspace_layout(cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I)
    assert lay["block_m"] == 160, lay  # the multi-launch call runs the block-tiled kernels too
    wts = weights(d, dev, fmt)
    got = persistent(d, cfg, dev, fmt, wts)
    ref = multi_launch(d, cfg, dev, fmt, wts)
    diff = np.argwhere(got != ref)
    assert diff.size == 0, "%s: %d elements differ, first %s" % (name, diff.shape[0], diff[:4].tolist())
    assert np.all(got[no_local_rows(cfg, d)] == 0)
    if fmt == w4.WEIGHTS_INT4_PACKED:  # and a few rows against the oracle itself
        rows = np.array([0, 1, cfg.T // 2, cfg.T - 1])
        assert_bf16_close(got[rows], oracle_rows_parallel(d, cfg, rows), "%s persistent" % name)


SMALL = {
    # name: (T, H, I, E_total, topk, expert_begin, E_local, seed), or a config
    "tiny": "tiny",
    "decode": "decode",
    "ragged": (700, 384, 256, 5, 2, 1, 3, 82),
    "one_expert": (300, 256, 128, 8, 3, 5, 1, 83),
    "many_pairs": (1500, 256, 128, 16, 4, 0, 8, 84),  # > 4096 pairs: the chunked align
    # H = 128 with top-32: a token's 32 slots sit in lanes the narrow column
    # loop leaves without columns (the combine phase's shuffles read them)
    "h128_top32": (160, 128, 128, 64, 32, 0, 32, 85),
    # the largest E_l: 1024 experts of ~16 rows, one mostly empty m-block each
    "many_experts": (2000, 256, 128, 1024, 8, 0, 1024, 86),
}


@pytest.mark.parametrize("case", list(SMALL))
@pytest.mark.parametrize("fmt", FORMATS)
def test_persistent_matches_oracle(dev, case, fmt):
    fp4 = fmt == w4.WEIGHTS_FP4_PACKED
    if isinstance(SMALL[case], str):
        cfg, d = moe_inputs(SMALL[case])
        d = with_fp4_weights(cfg, d) if fp4 else dict(d)
    else:
        T, H, I, Et, k, eb, El, seed = SMALL[case]
        gen = synth.random_moe_fp4 if fp4 else synth.random_moe
        cfg, d = gen(T, H, I, Et, k, eb, El, seed=seed)
    d["topk_ids"] = d["topk_ids"].copy()
    d["topk_ids"][:2] = -1  # tokens with no expert at all
    got = persistent(d, cfg, dev, fmt, weights(d, dev, fmt))
    rows = np.arange(cfg.T)
    ref = oracle_rows_parallel(d, cfg, rows, fn=oracle_fn(fmt))
    assert_bf16_close(got, ref, "persistent %s fmt %d" % (case, fmt))
    assert np.all(got[no_local_rows(cfg, d)] == 0)


def test_persistent_poisoned_workspace_and_reuse(dev):
    """One workspace, filled with 0xFF bytes (the barrier counter included),
    serves three calls of different shapes in a row (the largest first); the
    output buffer starts poisoned; each call must equal the oracle."""
    fmt = w4.WEIGHTS_INT4_PACKED
    cases = [synth.random_moe(1200, 256, 256, 16, 4, 0, 8, seed=91),   # chunked align
             synth.random_moe(40, 256, 256, 16, 4, 8, 8, seed=92),     # a few rows
             synth.random_moe(500, 256, 256, 16, 4, 4, 8, seed=93)]
    need = max(w4.fused_moe_persistent_workspace_bytes(c.T, c.H, c.topk, c.E_local, c.I, fmt)
               for c, _ in cases)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    out = torch.full((cases[0][0].T, 256), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
    for cfg, d in cases:
        o = out[:cfg.T]
        got = persistent(d, cfg, dev, fmt, weights(d, dev, fmt), out=o, workspace=ws)
        ref = oracle_rows_parallel(d, cfg, np.arange(cfg.T))
        assert not np.any(np.isnan(synth.bf16_bits_to_f32(got)))
        assert_bf16_close(got, ref, "reuse T=%d" % cfg.T)
        assert np.all(got[no_local_rows(cfg, d)] == 0)


def test_persistent_stage_events_bracket_the_call(dev):
    """The stage events are recorded around the two launches: the gate_up,
    down and combine spans (3, 4 and 5 all after the single launch) read 0
    for down and combine."""
    cfg, d = synth.random_moe(256, 256, 128, 8, 2, 0, 4, seed=94)
    fmt = w4.WEIGHTS_INT4_PACKED
    wts = weights(d, dev, fmt)
    # sized before arming: a workspace query consumes the arming too
    need = w4.fused_moe_persistent_workspace_bytes(cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I, fmt)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    timer = w4.StageTimer()
    try:
        timer.arm()
        got = persistent(d, cfg, dev, fmt, wts, workspace=ws)
        ms = timer.read_ms()
    finally:
        timer.close()
    assert all(v >= 0 for v in ms.values()), ms
    assert ms["gate_up"] > 0 and ms["down"] < 0.005 and ms["combine"] < 0.005, ms
    assert_bf16_close(got, oracle_rows_parallel(d, cfg, np.arange(cfg.T)), "events")


def test_persistent_graph_replays_match_eager(dev):
    """The single launch recorded into a HIP graph (the align clears the
    barrier counter on every replay): replays with the other input set copied
    into the captured buffers, and eager work between them, equal the eager
    calls bit for bit."""
    fmt = w4.WEIGHTS_INT4_PACKED
    cfg, d = synth.random_moe(512, 256, 256, 8, 2, 0, 4, seed=95)
    _, d2 = synth.random_moe(512, 256, 256, 8, 2, 0, 4, seed=96)
    wts = weights(d, dev, fmt)
    need = w4.fused_moe_persistent_workspace_bytes(cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I, fmt)
    refs = [persistent(dd, cfg, dev, fmt, wts) for dd in (d, d2)]
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    hid, ids, tw = bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev), dput(d["topk_weights"], dev)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            w4.fused_moe_persistent(hid, ids, tw, cfg.expert_begin, cfg.E_local, cfg.I, wts, fmt,
                                    out=out, workspace=ws)
    junk = torch.randn(1 << 20, device=dev)
    for r in range(4):
        src = (d, d2)[r % 2]
        hid.copy_(bf16_dev(src["hidden"], dev))
        ids.copy_(dput(src["topk_ids"], dev))
        tw.copy_(dput(src["topk_weights"], dev))
        out.fill_(-1.0)
        junk.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_host(out), refs[r % 2]), "replay %d" % r
