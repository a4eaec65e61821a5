"""The fused forward with a caller's bound on the local pairs
(w4a8_fused_moe_bounded), through the C ABI.

* Within the bound, on a shape whose path the bound does not change (decode:
  16-row m-blocks either way), the output is bit-identical to the unbounded
  export of the same weight format (canonical int4, prepacked int4, fp4), and
  the call reports the local pair count.
* Where the counts decide the path on the device (the align's cost model:
  per-expert 16 / 32-row skinny blocks or the block-tiled kernels), the call
  reports the path it took, the clear cases take the expected one, and both
  are held to the oracle's bar; the unbounded export chooses the same way
  between its two host rules (its path flag read from the workspace).
* Beyond the bound nothing is computed: every output row is +0 (the output
  starts poisoned), the reported count is the real one, and the same
  workspace then serves a call within the bound (single-block align for few
  pairs, the chunked count/scan/scatter align for many).
"""
import numpy as np
import pytest
import torch

import oracle
from w4a8_moe_grouped_amd import lib as w4
from w4a8_moe_grouped_amd import synth

from test_gpu_parity import assert_bf16_close, bf16_dev, bf16_host, dput, oracle_rows_parallel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    w4.load()
    return torch.device("cuda:0")


def local_pairs_of(cfg, d):
    ids = d["topk_ids"]
    return int(np.sum((ids >= cfg.expert_begin) & (ids < cfg.expert_begin + cfg.E_local)))


def weights(d, dev, fmt):
    if fmt == w4.WEIGHTS_INT4:
        return tuple(dput(d[k], dev) for k in ("w13", "s13", "w2", "s2"))
    if fmt == w4.WEIGHTS_INT4_PACKED:
        return w4.prepack_weights(dput(d["w13"], dev), dput(d["s13"], dev)) + \
            w4.prepack_weights(dput(d["w2"], dev), dput(d["s2"], dev))
    return w4.prepack_weights_fp4(dput(d["w13"], dev), dput(d["s13"], dev), w4.FP4_GATE_UP) + \
        w4.prepack_weights_fp4(dput(d["w2"], dev), dput(d["s2"], dev), w4.FP4_DOWN)


def unbounded(d, cfg, dev, fmt, ws):
    hid = bf16_dev(d["hidden"], dev)
    ids, wts = dput(d["topk_ids"], dev), dput(d["topk_weights"], dev)
    if fmt == w4.WEIGHTS_FP4_PACKED:
        return w4.fused_moe_fp4(hid, ids, wts, cfg.expert_begin, cfg.E_local, cfg.I, ws)
    canon = tuple(dput(d[k], dev) for k in ("w13", "s13", "w2", "s2")) \
        if fmt == w4.WEIGHTS_INT4 else None
    if fmt == w4.WEIGHTS_INT4:
        return w4.fused_moe(hid, ids, wts, cfg.expert_begin, cfg.E_local, *canon)
    shapes = (torch.empty((cfg.E_local, 2 * cfg.I, cfg.H // 2), dtype=torch.uint8, device=dev),
              torch.empty((cfg.E_local, 2 * cfg.I, cfg.H // 128), dtype=torch.float32, device=dev),
              torch.empty((cfg.E_local, cfg.H, cfg.I // 2), dtype=torch.uint8, device=dev),
              torch.empty((cfg.E_local, cfg.H, cfg.I // 128), dtype=torch.float32, device=dev))
    return w4.fused_moe(hid, ids, wts, cfg.expert_begin, cfg.E_local, *shapes, prepacked=ws)


def bounded(d, cfg, dev, fmt, ws, bound, out=None, workspace=None):
    out, n = w4.fused_moe_bounded(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev),
                                  dput(d["topk_weights"], dev), cfg.expert_begin, cfg.E_local, cfg.I,
                                  ws, fmt, bound, out=out, workspace=workspace)
    torch.cuda.synchronize()
    n = n.cpu().numpy()
    bounded.last_path = int(n[1])
    return out, int(n[0])


@pytest.mark.parametrize("fmt", [w4.WEIGHTS_INT4, w4.WEIGHTS_INT4_PACKED, w4.WEIGHTS_FP4_PACKED])
def test_bounded_equals_unbounded_decode(dev, fmt):
    gen = synth.random_moe_fp4 if fmt == w4.WEIGHTS_FP4_PACKED else synth.random_moe
    cfg, d = gen(64, 7168, 2048, 256, 8, 0, 32, seed=101)
    P = local_pairs_of(cfg, d)
    print("bounded decode: fmt=%d T=64 P=%d" % (fmt, P), flush=True)
    ws = weights(d, dev, fmt)
    ref = unbounded(d, cfg, dev, fmt, ws)
    torch.cuda.synchronize()
    for bound in (P, P + 37, 64 * 8, 1 << 20):
        got, n = bounded(d, cfg, dev, fmt, ws, bound)
        assert n == P
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), bound


# single-block align and 16-row blocks / chunked align and the path chosen on the device
@pytest.mark.parametrize("T,seed", [(64, 102), (2048, 103)])
def test_bounded_overflow_writes_zeros_then_recovers(dev, T, seed):
    cfg, d = synth.random_moe(T, 7168, 2048, 256, 8, 0, 32, seed=seed)
    P = local_pairs_of(cfg, d)
    print("bounded overflow: T=%d P=%d" % (T, P), flush=True)
    ws = weights(d, dev, w4.WEIGHTS_INT4_PACKED)
    need = w4.fused_moe_bounded_workspace_bytes(T, cfg.H, cfg.topk, cfg.E_local, cfg.I, P - 1)
    work = torch.full((need,), 0x5A, dtype=torch.uint8, device=dev)
    out = torch.full((T, cfg.H), 1.0, dtype=torch.bfloat16, device=dev)
    out, n = bounded(d, cfg, dev, w4.WEIGHTS_INT4_PACKED, ws, P - 1, out=out, workspace=work)
    assert n == P
    assert torch.count_nonzero(out.view(torch.int16)).item() == 0
    # the same workspace, a bound that fits the same count: a normal call
    # (sizes for P - 1 pairs hold a call bounded by P - 1; run a smaller
    # routing that fits: the first tokens only)
    t2 = max(1, T // 2)
    while True:
        sub = {k: d[k][:t2] for k in ("hidden", "topk_ids", "topk_weights")}
        sub.update({k: d[k] for k in ("w13", "s13", "w2", "s2")})
        P2 = local_pairs_of(cfg, sub)
        if P2 <= P - 1:
            break
        t2 //= 2
    cfg2 = synth.MoEConfig("adhoc", T=t2, H=cfg.H, I=cfg.I, E_total=cfg.E_total, topk=cfg.topk,
                           expert_begin=cfg.expert_begin, E_local=cfg.E_local, seed=seed)
    out2, n2 = bounded(sub, cfg2, dev, w4.WEIGHTS_INT4_PACKED, ws, P - 1, workspace=work)
    assert n2 == P2
    rows = np.arange(t2) if t2 <= 64 else np.linspace(0, t2 - 1, 48).astype(np.int64)
    ref = oracle_rows_parallel(sub, cfg2, rows)
    assert_bf16_close(bf16_host(out2)[rows], ref, "bounded after overflow (T=%d, P=%d)" % (t2, P2))


def first_last_tokens(cfg, d):
    rows = set()
    for e in range(cfg.E_local):  # the first and the last token of every local expert
        toks = np.nonzero(np.any(d["topk_ids"] == e + cfg.expert_begin, axis=1))[0]
        if toks.size:
            rows.update((int(toks[0]), int(toks[-1])))
    return np.array(sorted(rows))


@pytest.mark.parametrize("T,E_total,routing,slack,want", [
    (512, 256, "uniform", 1.05, 0),   # ~16 pairs per expert: skinny 16 / 32-row blocks
    (512, 256, "uniform", 4.1, 0),    # a loose bound: the counts still decide
    (512, 32, "uniform", 1.02, 1),    # every expert local, ~128 pairs each: block-tiled
    (256, 256, "zipf_id", 1.02, 0),   # skewed, 5..250 pairs per expert: skinny
])
def test_bounded_paths_match_oracle(dev, T, E_total, routing, slack, want):
    cfg, d = synth.random_moe(T, 7168, 2048, E_total, 8, 0, 32, seed=104, routing=routing)
    P = local_pairs_of(cfg, d)
    bound = int(P * slack) + 1
    print("bounded path: T=%d E=%d %s P=%d bound=%d" % (T, E_total, routing, P, bound), flush=True)
    ws = weights(d, dev, w4.WEIGHTS_INT4_PACKED)
    got, n = bounded(d, cfg, dev, w4.WEIGHTS_INT4_PACKED, ws, bound)
    assert n == P
    assert bounded.last_path == want
    got = bf16_host(got)
    rows = first_last_tokens(cfg, d)
    ref = oracle_rows_parallel(d, cfg, rows)
    assert_bf16_close(got[rows], ref, "bounded T=%d %s bound=%d path %d (%d tokens)"
                      % (T, routing, bound, want, rows.size))
    ids = d["topk_ids"]
    none_local = ~np.any((ids >= 0) & (ids < cfg.E_local), axis=1)
    assert np.all(got[none_local] == 0)


@pytest.mark.parametrize("T,E_total,routing,want", [
    (512, 32, "uniform", 1),    # T*topk/E_l = 128: between the host rules; ~128 real rows: tiled
    (256, 256, "zipf_id", 0),   # T*topk/E_l = 64; 5..250 real rows: skinny
])
def test_unbounded_device_path_choice(dev, T, E_total, routing, want):
    cfg, d = synth.random_moe(T, 7168, 2048, E_total, 8, 0, 32, seed=105, routing=routing)
    lay = w4.fused_moe_workspace_layout(T, cfg.H, cfg.topk, cfg.E_local, cfg.I)
    assert lay["device_path"] and lay["two_lists"]
    ws = torch.zeros(w4.fused_moe_workspace_bytes(T, cfg.H, cfg.topk, cfg.E_local, cfg.I),
                     dtype=torch.uint8, device=dev)
    print("unbounded device path: T=%d E=%d %s" % (T, E_total, routing), flush=True)
    packed = weights(d, dev, w4.WEIGHTS_INT4_PACKED)
    out = unbounded_with_workspace(d, cfg, dev, packed, ws)
    torch.cuda.synchronize()
    path = int(ws[lay["path"]:lay["path"] + 4].view(torch.int32).item())
    assert path == want
    got = bf16_host(out)
    rows = first_last_tokens(cfg, d)
    ref = oracle_rows_parallel(d, cfg, rows)
    assert_bf16_close(got[rows], ref, "unbounded T=%d %s device path %d (%d tokens)"
                      % (T, routing, path, rows.size))


def unbounded_with_workspace(d, cfg, dev, packed, ws):
    shapes = (torch.empty((cfg.E_local, 2 * cfg.I, cfg.H // 2), dtype=torch.uint8, device=dev),
              torch.empty((cfg.E_local, 2 * cfg.I, cfg.H // 128), dtype=torch.float32, device=dev),
              torch.empty((cfg.E_local, cfg.H, cfg.I // 2), dtype=torch.uint8, device=dev),
              torch.empty((cfg.E_local, cfg.H, cfg.I // 128), dtype=torch.float32, device=dev))
    return w4.fused_moe(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev),
                        dput(d["topk_weights"], dev), cfg.expert_begin, cfg.E_local, *shapes,
                        workspace=ws, prepacked=packed)


@pytest.mark.parametrize("fmt,E_total,routing,want", [
    (w4.WEIGHTS_FP4_PACKED, 32, "uniform", 1),   # fp4 weights, ~128 rows per expert: tiled
    (w4.WEIGHTS_FP4_PACKED, 256, "zipf_id", 0),  # fp4 weights, skewed: skinny
    (w4.WEIGHTS_INT4, 32, "uniform", 1),         # canonical int4 layout on the tiled kernels
])
def test_device_path_choice_weight_formats(dev, fmt, E_total, routing, want):
    """The device-chosen path with the other weight formats, bounded by the
    exact local pair count, against the oracle of the same format."""
    T = 512 if routing == "uniform" else 256
    gen = synth.random_moe_fp4 if fmt == w4.WEIGHTS_FP4_PACKED else synth.random_moe
    cfg, d = gen(T, 7168, 2048, E_total, 8, 0, 32, seed=106, routing=routing)
    P = local_pairs_of(cfg, d)
    print("device path, format %d: T=%d E=%d %s P=%d" % (fmt, T, E_total, routing, P), flush=True)
    ws = weights(d, dev, fmt)
    got, n = bounded(d, cfg, dev, fmt, ws, P)
    assert n == P and bounded.last_path == want
    rows = first_last_tokens(cfg, d)
    fn = oracle.fused_moe_fp4 if fmt == w4.WEIGHTS_FP4_PACKED else None
    ref = oracle_rows_parallel(d, cfg, rows, fn=fn)
    assert_bf16_close(bf16_host(got)[rows], ref, "format %d %s path %d (%d tokens)" % (fmt, routing, want, rows.size))
