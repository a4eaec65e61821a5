"""GPU parity of the fp4-weight forward (FP4 E2M1 weights with per-32-K
UE8M0 scales, DeepGEMM PR #53 "Changes") against the CPU oracle.

* w4a8_prepack_weights_fp4 is pure data movement: its output must equal, byte
  for byte, the layout written out here with numpy (the int4 blocking, the
  gate_up role's nibble order k0,k2,k4,k6,k1,k3,k5,k7 inside each dword, the
  scale dwords in the fp32-scale positions, zero past the last group).
* w4a8_fused_moe_fp4_prepacked against oracle.fused_moe_fp4 at the same bar as
  the int4 path (relative Frobenius <= 1e-3, max |diff| <= 2e-2 max|ref|,
  rows with no local pair exactly +0), on the decode (skinny) and the
  block-tiled paths, ragged shapes and the degenerate routings.
"""
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


def numpy_layout_fp4(w, sb, role):
    E, N, K2 = w.shape
    G = K2 // 64
    G4 = (G + 3) // 4
    if role == w4.FP4_GATE_UP:
        d = w.reshape(-1).view(np.uint32)
        out = np.zeros_like(d)
        for i, src in enumerate((0, 2, 4, 6, 1, 3, 5, 7)):
            out |= ((d >> np.uint32(4 * src)) & np.uint32(0xF)) << np.uint32(4 * i)
        w = out.view(np.uint8).reshape(E, N, K2)
    wp = w.reshape(E, N // 16, 16, G, 64).transpose(0, 1, 3, 2, 4).reshape(E, -1)
    dw = np.ascontiguousarray(sb).view(np.uint32).reshape(E, N, G)
    sp = np.zeros((E, N, G4 * 4), np.uint32)
    sp[:, :, :G] = dw
    sp = sp.reshape(E, N // 16, 16, G4, 4).transpose(0, 1, 3, 2, 4).reshape(E, -1)
    return wp, sp


@pytest.mark.parametrize("role", [0, 1])
@pytest.mark.parametrize("E,N,K", [(1, 16, 128), (3, 48, 640), (2, 64, 384)])
def test_prepack_fp4_layout_bit_exact(dev, role, E, N, K):
    rng = np.random.default_rng(E * 100 + N + K + role)
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    sb = rng.integers(0, 256, size=(E, N, K // 32), dtype=np.uint8)
    wp, sp = w4.prepack_weights_fp4(dput(w, dev), dput(sb, dev), role)
    torch.cuda.synchronize()
    ew, es = numpy_layout_fp4(w, sb, role)
    assert np.array_equal(wp.cpu().numpy(), ew)
    assert np.array_equal(sp.cpu().numpy().view(np.uint32), es)


def fp4_case(case):
    if case == "tiny":
        return synth.random_moe_fp4(16, 256, 128, 4, 2, 0, 4, seed=0)
    if case == "decode":
        cfg = synth.CONFIGS["decode"]
        return cfg, synth.gen_moe_fp4(cfg)
    if case == "tile_small":       # block-tiled path
        return synth.random_moe_fp4(512, 256, 256, 8, 2, 0, 4, seed=31)
    if case == "tile_ragged":      # H = 384: a partial weight block; 3 and 1 K-groups
        return synth.random_moe_fp4(700, 384, 128, 5, 2, 1, 3, seed=32)
    if case == "single_token":
        return synth.random_moe_fp4(1, 7168, 2048, 64, 8, 0, 16, seed=22)
    if case == "five_groups":      # 5 and 3 K-groups: padded scale blocks
        return synth.random_moe_fp4(24, 640, 384, 8, 2, 2, 4, seed=41)
    if case == "k1_e1":
        return synth.random_moe_fp4(40, 384, 128, 1, 1, 0, 1, seed=23)
    if case == "two_slices":       # ~30 rows per expert: 32-row blocks with both 16-row slices
        return synth.random_moe_fp4(120, 256, 128, 4, 1, 0, 4, seed=42)
    assert case == "all_non_local"
    cfg, d = synth.random_moe_fp4(48, 256, 128, 8, 2, 4, 4, seed=27)
    d["topk_ids"][:] = d["topk_ids"] % 4
    return cfg, d


@pytest.mark.parametrize("case", ["tiny", "decode", "tile_small", "tile_ragged", "single_token",
                                  "five_groups", "k1_e1", "two_slices", "all_non_local"])
def test_fused_moe_fp4_matches_oracle(dev, case):
    cfg, d = fp4_case(case)
    packed = w4.prepack_weights_fp4(dput(d["w13"], dev), dput(d["s13"], dev), w4.FP4_GATE_UP) + \
        w4.prepack_weights_fp4(dput(d["w2"], dev), dput(d["s2"], dev), w4.FP4_DOWN)
    out = w4.fused_moe_fp4(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev),
                           dput(d["topk_weights"], dev), cfg.expert_begin, cfg.E_local, cfg.I, packed)
    torch.cuda.synchronize()
    got = bf16_host(out)
    rows = np.arange(cfg.T) if cfg.T <= 64 or case == "tile_small" else \
        np.unique(np.linspace(0, cfg.T - 1, 40).astype(np.int64))
    ref = oracle.fused_moe_fp4(d["hidden"][rows], d["topk_ids"][rows], d["topk_weights"][rows],
                               cfg.expert_begin, cfg.E_local, d["w13"], d["s13"], d["w2"], d["s2"])
    assert_bf16_close(got[rows], ref, "fp4 " + case)
    ids = d["topk_ids"]
    none_local = ~np.any((ids >= cfg.expert_begin) & (ids < cfg.expert_begin + cfg.E_local), axis=1)
    assert np.all(got[none_local] == 0)
