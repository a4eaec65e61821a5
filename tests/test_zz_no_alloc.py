"""The allocation-free fused forward (w4a8_fused_moe_prepacked_noalloc)
against the workspace export it varies (w4a8_fused_moe_prepacked), through
the C ABI: the same kernels, so the outputs must be bit-identical.  Two calls
in a row on the library's own scratch array, the second with fewer tokens and
other routing (the array keeps the first call's contents), then a shape that
needs more scratch than the array holds is rejected before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

from w4a8_moe_grouped_amd import lib as w4
from w4a8_moe_grouped_amd import synth

pytestmark = pytest.mark.gpu


def dput(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def test_noalloc_equals_workspace_export_twice():
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    w4.load()
    # decode at the model's sizes (64 tokens, 32 of 256 experts, top-8), then
    # 13 tokens with other routing on the same weights
    cfg1, d1 = synth.random_moe(64, 7168, 2048, 256, 8, 0, 32, seed=91)
    cfg2, d2 = synth.random_moe(13, 7168, 2048, 256, 8, 0, 32, seed=92)
    d2["topk_ids"][:3] = -1
    packed = w4.prepack_weights(dput(d1["w13"], dev), dput(d1["s13"], dev)) + \
        w4.prepack_weights(dput(d1["w2"], dev), dput(d1["s2"], dev))
    w13, s13, w2, s2 = (dput(d1[k], dev) for k in ("w13", "s13", "w2", "s2"))
    for cfg, d in ((cfg1, d1), (cfg2, d2)):
        hid = dput(d["hidden"].view(np.int16), dev).view(torch.bfloat16)
        ids, wts = dput(d["topk_ids"], dev), dput(d["topk_weights"], dev)
        print("noalloc: T=%d H=%d I=%d topk=%d" % (cfg.T, cfg.H, cfg.I, cfg.topk), flush=True)
        got = w4.fused_moe_noalloc(hid, ids, wts, cfg.expert_begin, cfg.E_local, cfg.I, packed)
        ref = w4.fused_moe(hid, ids, wts, cfg.expert_begin, cfg.E_local, w13, s13, w2, s2,
                           prepacked=packed)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), cfg.T


def test_noalloc_rejects_shapes_beyond_its_scratch():
    L = w4.load()
    bogus = ctypes.c_void_p(0x1000)
    # 4096 tokens x top-8 at H = 7168, I = 2048 needs ~1 GB of intermediates
    rc = L.w4a8_fused_moe_prepacked_noalloc(bogus, 4096, 7168, bogus, bogus, 8, 0, 32, 2048,
                                            bogus, bogus, bogus, bogus, bogus, None)
    assert rc == 3  # W4A8_ERR_WORKSPACE, nothing launched
