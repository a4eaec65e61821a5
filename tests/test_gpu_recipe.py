"""GPU parity of the finer activation-scale recipes (DeepGEMM PR #53 commit
notes: per-32 and 128/64 activation scales): the SwiGLU output requantised
per 64 or 32 K, each block promoted with its own scale in the down GEMM,
against the oracle's fused_moe_recipe at the usual bar, for int4 and fp4
weights; and the requantised intermediate's codes and block scales read
back from the workspace."""
import numpy as np
import pytest
import torch

import oracle
from w4a8_moe_grouped_amd import lib as w4
from w4a8_moe_grouped_amd import synth

from test_gpu_parity import assert_bf16_close, bf16_dev, bf16_host, dput

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    w4.load()
    return torch.device("cuda:0")


def packed(d, fp4, dev):
    w = [dput(d[k], dev) for k in ("w13", "s13", "w2", "s2")]
    if fp4:
        return w4.prepack_weights_fp4(w[0], w[1], w4.FP4_GATE_UP) + w4.prepack_weights_fp4(w[2], w[3], w4.FP4_DOWN)
    return w4.prepack_weights(w[0], w[1]) + w4.prepack_weights(w[2], w[3])


CASES = {
    "decode": lambda gen: (synth.CONFIGS["decode"], (synth.gen_moe_fp4 if gen is synth.random_moe_fp4
                                                      else synth.gen_moe)(synth.CONFIGS["decode"])),
    "nt2": lambda gen: gen(24, 512, 256, 8, 2, 0, 2, seed=61),       # 32-row m-blocks (F/E = 24)
    "nt4": lambda gen: gen(300, 256, 256, 8, 2, 0, 4, seed=62),      # 64-row m-blocks (F/E = 150)
    "ragged": lambda gen: gen(24, 640, 384, 8, 2, 2, 4, seed=63),    # 5 and 3 K-groups
}


@pytest.mark.parametrize("group", [64, 32])
@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("case", list(CASES))
def test_fused_moe_recipe_matches_oracle(dev, case, fp4, group):
    gen = synth.random_moe_fp4 if fp4 else synth.random_moe
    cfg, d = CASES[case](gen)
    T, H, k, E, I = cfg.T, cfg.H, cfg.topk, cfg.E_local, cfg.I
    ws = torch.zeros(w4.fused_moe_workspace_bytes(T, H, k, E, I), dtype=torch.uint8, device=dev)
    out = w4.fused_moe_recipe(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev), dput(d["topk_weights"], dev),
                              cfg.expert_begin, E, I, packed(d, fp4, dev),
                              w4.WEIGHTS_FP4_PACKED if fp4 else w4.WEIGHTS_INT4_PACKED, group, workspace=ws)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 64 else np.linspace(0, T - 1, 40).astype(np.int64)
    ref, inter = oracle.fused_moe_recipe(d["hidden"][rows], d["topk_ids"][rows], d["topk_weights"][rows],
                                         cfg.expert_begin, E, d["w13"], d["s13"], d["w2"], d["s2"], group,
                                         fp4=fp4, intermediates=True)
    assert_bf16_close(bf16_host(out)[rows], ref, "%s %s per-%d" % (case, "fp4" if fp4 else "int4", group))
    if case == "decode":
        # the requantised intermediate's block scales (all rows were run)
        lay = w4.fused_moe_workspace_layout(T, H, k, E, I)
        wsh = ws.cpu().numpy()
        P = inter["qh"].shape[0]
        side = wsh[lay["qh_side"]:lay["qh_side"] + 8 * P * (I // group)].view(np.float32).reshape(P, -1, 2)
        scale = side[:, :, 0] / np.float32(512)
        rel = np.max(np.abs(scale.astype(np.float64) - inter["sh"]) / inter["sh"])
        print("per-%d %s: scale max rel %.1e" % (group, "fp4" if fp4 else "int4", rel))
        assert rel <= 2e-6


@pytest.mark.parametrize("fp4", [False, True])
def test_recipe_degenerate_routings(dev, fp4):
    """No local pair at all (output +0) and T = 0 (nothing launched)."""
    gen = synth.random_moe_fp4 if fp4 else synth.random_moe
    cfg, d = gen(48, 256, 128, 8, 2, 4, 4, seed=64)
    d["topk_ids"][:] = d["topk_ids"] % 4          # every id below expert_begin
    fmt = w4.WEIGHTS_FP4_PACKED if fp4 else w4.WEIGHTS_INT4_PACKED
    out = w4.fused_moe_recipe(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev), dput(d["topk_weights"], dev),
                              cfg.expert_begin, cfg.E_local, cfg.I, packed(d, fp4, dev), fmt, 32)
    torch.cuda.synchronize()
    assert np.all(bf16_host(out) == 0)
    empty = torch.empty((0, cfg.H), dtype=torch.bfloat16, device=dev)
    o0 = w4.fused_moe_recipe(empty, torch.empty((0, 2), dtype=torch.int32, device=dev),
                             torch.empty((0, 2), dtype=torch.float32, device=dev), cfg.expert_begin,
                             cfg.E_local, cfg.I, packed(d, fp4, dev), fmt, 64)
    assert o0.shape == (0, cfg.H)
