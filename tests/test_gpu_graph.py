"""The fused forward captured in a HIP graph (torch.cuda.CUDAGraph on ROCm)
and replayed: every replay must equal the eager call on the same inputs, bit
for bit, with the program's own eager work and synchronisations between the
replays and new inputs copied into the captured buffers before each one.
(The library records no memset, allocation or synchronisation, so a call is
capturable as it is.)"""
import numpy as np
import pytest
import torch

from w4a8_moe_grouped_amd import lib as w4
from w4a8_moe_grouped_amd import synth

from test_gpu_parity import bf16_dev, dput

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    w4.load()
    return torch.device("cuda:0")


def _inputs(cfg, d, dev):
    return (bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev), dput(d["topk_weights"], dev))


@pytest.mark.parametrize("fmt", ["int4", "int4_prepacked", "fp4"])
@pytest.mark.parametrize("shape", ["decode_like", "tile"])
def test_graph_replays_match_eager(dev, fmt, shape):
    gen = synth.random_moe_fp4 if fmt == "fp4" else synth.random_moe
    if shape == "tile":
        args = (512, 256, 256, 8, 2, 0, 4)
    else:
        args = (64, 1024, 512, 64, 8, 0, 16)
    cfg, d = gen(*args, seed=5)
    _, d2 = gen(*args, seed=6)          # second set of activations/routing
    wts = [dput(d[k], dev) for k in ("w13", "s13", "w2", "s2")]
    if fmt == "fp4":
        packed = w4.prepack_weights_fp4(wts[0], wts[1], w4.FP4_GATE_UP) + \
            w4.prepack_weights_fp4(wts[2], wts[3], w4.FP4_DOWN)
    elif fmt == "int4_prepacked":
        packed = w4.prepack_weights(wts[0], wts[1]) + w4.prepack_weights(wts[2], wts[3])
    T, H, k, E, I = cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I
    ws = torch.empty(w4.fused_moe_workspace_bytes(T, H, k, E, I), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def call(hid, ids, tw, o, w):
        if fmt == "fp4":
            return w4.fused_moe_fp4(hid, ids, tw, cfg.expert_begin, E, I, packed, out=o, workspace=w)
        return w4.fused_moe(hid, ids, tw, cfg.expert_begin, E, *wts, out=o, workspace=w,
                            prepacked=packed if fmt == "int4_prepacked" else None)

    hid, ids, tw = _inputs(cfg, d, dev)
    # eager references for both input sets (own workspace and output)
    ws_e = torch.empty_like(ws)
    refs = []
    for dd in (d, d2):
        o = torch.empty_like(out)
        call(*_inputs(cfg, dd, dev), o, ws_e)
        torch.cuda.synchronize()
        refs.append(o.clone())
    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(hid, ids, tw, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(hid, ids, tw, out, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        dd = (d, d2)[rep % 2]
        h2, i2, t2 = _inputs(cfg, dd, dev)
        hid.copy_(h2)
        ids.copy_(i2)
        tw.copy_(t2)
        out.fill_(0)
        g.replay()
        # the program's own eager work between replays
        junk = torch.empty_like(out)
        call(h2, i2, t2, junk, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), refs[rep % 2].view(torch.int16)), "replay %d" % rep
        assert torch.equal(junk.view(torch.int16), refs[rep % 2].view(torch.int16))
    del g
