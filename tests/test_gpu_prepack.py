"""GPU checks of the prepacked weight layout and the fused forward on it.

* w4a8_prepack_weights is pure data movement: its output must equal, byte for
  byte, the layout written out here with numpy reshapes (weights
  [E][N/16][G][16][64 B], scales [E][N/16][ceil(G/4)][16][4], zero past the
  last group of a row).
* w4a8_fused_moe_prepacked runs the same kernels with other addresses, so its
  output must be bit-identical to w4a8_fused_moe on the canonical weights, and
  within the usual bar of the oracle.
"""
import numpy as np
import pytest
import torch
import oracle

from w4a8_moe_grouped_amd import lib as w4
from w4a8_moe_grouped_amd import synth

from test_gpu_parity import (assert_bf16_close, bf16_dev, bf16_host, dput, moe_inputs,
                             oracle_rows, tile_case)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    w4.load()
    return torch.device("cuda:0")


def numpy_layout(w, s):
    """The prepacked layout by reshapes: w [E, N, K/2] u8, s [E, N, G] f32."""
    E, N, K2 = w.shape
    G = K2 // 64
    G4 = (G + 3) // 4
    wp = w.reshape(E, N // 16, 16, G, 64).transpose(0, 1, 3, 2, 4).reshape(E, -1)
    sp = np.zeros((E, N, G4 * 4), dtype=np.float32)
    sp[:, :, :G] = s
    sp = sp.reshape(E, N // 16, 16, G4, 4).transpose(0, 1, 3, 2, 4).reshape(E, -1)
    return wp, sp


@pytest.mark.parametrize("E,N,K", [(1, 16, 128), (2, 32, 256), (3, 48, 640), (2, 64, 384),
                                   (4, 256, 7168)])
def test_prepack_layout_bit_exact(dev, E, N, K):
    rng = np.random.default_rng(E * 1000 + N + K)
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    s = rng.standard_normal((E, N, K // 128)).astype(np.float32)
    wp, sp = w4.prepack_weights(dput(w, dev), dput(s, dev))
    torch.cuda.synchronize()
    ew, es = numpy_layout(w, s)
    assert np.array_equal(wp.cpu().numpy(), ew)
    assert np.array_equal(sp.cpu().numpy().view(np.uint32), es.view(np.uint32))


def run_both(cfg, d, dev):
    w13, s13 = dput(d["w13"], dev), dput(d["s13"], dev)
    w2, s2 = dput(d["w2"], dev), dput(d["s2"], dev)
    args = (bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev), dput(d["topk_weights"], dev),
            cfg.expert_begin, cfg.E_local, w13, s13, w2, s2)
    canon = w4.fused_moe(*args)
    packed = w4.fused_moe(*args, prepacked=w4.prepack_weights(w13, s13) + w4.prepack_weights(w2, s2))
    torch.cuda.synchronize()
    return bf16_host(canon), bf16_host(packed)


def prepacked_case(case):
    if case in ("tiny", "decode"):
        return moe_inputs(case)
    if case.startswith("tile_"):
        return tile_case(case)
    if case == "single_token":
        return synth.random_moe(1, 7168, 2048, 256, 8, 0, 256, seed=22)
    if case == "k1_e1":
        return synth.random_moe(40, 384, 128, 1, 1, 0, 1, seed=23)
    if case == "five_groups":       # K-groups 5 (gate_up) and 3 (down): padded scale blocks
        return synth.random_moe(24, 640, 384, 8, 2, 2, 4, seed=41)
    assert case == "all_non_local"
    cfg, d = synth.random_moe(48, 256, 128, 8, 2, 4, 4, seed=27)
    d["topk_ids"][:] = d["topk_ids"] % 4
    return cfg, d


@pytest.mark.parametrize("case", ["tiny", "decode", "tile_small", "tile_ragged", "single_token",
                                  "k1_e1", "five_groups", "all_non_local"])
def test_fused_moe_prepacked_matches_canonical(dev, case):
    cfg, d = prepacked_case(case)
    canon, packed = run_both(cfg, d, dev)
    assert np.array_equal(canon, packed), "prepacked path differs from the canonical one"
    rows = np.arange(cfg.T) if cfg.T <= 256 else np.linspace(0, cfg.T - 1, 48).astype(np.int64)
    assert_bf16_close(packed[rows], oracle_rows(d, cfg, rows), case)


def test_prepack_bf16_scales_equals_widened_fp32(dev):
    """bf16 checkpoint scales: the prepacked output equals the fp32 prepack of
    the same scales widened by torch (exact), byte for byte."""
    rng = np.random.default_rng(5)
    E, N, K = 3, 48, 640
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    s16 = torch.from_numpy(rng.uniform(0.002, 0.02, size=(E, N, K // 128)).astype(np.float32)).to(
        torch.bfloat16).to(dev)
    wd = dput(w, dev)
    a = w4.prepack_weights(wd, s16)
    b = w4.prepack_weights(wd, s16.to(torch.float32))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_fused_moe_with_bf16_checkpoint_scales(dev):
    """The forward on bf16-scale weights equals the oracle run on the same
    scales in fp32."""
    cfg, d = synth.random_moe(40, 384, 256, 8, 2, 0, 4, seed=43)
    for k in ("s13", "s2"):
        d[k] = torch.from_numpy(d[k]).to(torch.bfloat16).to(torch.float32).numpy()
    w13, w2 = dput(d["w13"], dev), dput(d["w2"], dev)
    s13 = torch.from_numpy(d["s13"]).to(torch.bfloat16).to(dev)
    s2 = torch.from_numpy(d["s2"]).to(torch.bfloat16).to(dev)
    packed = w4.prepack_weights(w13, s13) + w4.prepack_weights(w2, s2)
    out = w4.fused_moe(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev), dput(d["topk_weights"], dev),
                       cfg.expert_begin, cfg.E_local, w13, dput(d["s13"], dev), w2, dput(d["s2"], dev),
                       prepacked=packed)
    torch.cuda.synchronize()
    assert_bf16_close(bf16_host(out), oracle_rows(d, cfg, np.arange(cfg.T)), "bf16 scales")


@pytest.mark.parametrize("shape", ["skinny", "tile"])
@pytest.mark.parametrize("which", ["a1", "a2", "both"])
def test_fused_moe_static_activation_scales(dev, shape, which):
    """Static per-tensor activation scales (a checkpoint's input scales)
    against the oracle; the a2 scale is set low enough that some of the
    SwiGLU output saturates at 448 * s."""
    if shape == "tile":
        cfg, d = synth.random_moe(512, 256, 256, 8, 2, 0, 4, seed=45)
    else:
        cfg, d = synth.random_moe(48, 1024, 512, 16, 4, 0, 8, seed=46)
    _, inter = oracle.fused_moe(d["hidden"], d["topk_ids"], d["topk_weights"], cfg.expert_begin,
                                cfg.E_local, d["w13"], d["s13"], d["w2"], d["s2"], intermediates=True)
    a1 = float(np.float32(np.abs(synth.bf16_bits_to_f32(d["hidden"])).max() / 448.0))
    a2 = float(np.float32(np.median(inter["sh"])))
    a1 = a1 if which in ("a1", "both") else None
    a2 = a2 if which in ("a2", "both") else None
    w13, w2 = dput(d["w13"], dev), dput(d["w2"], dev)
    s13, s2 = dput(d["s13"], dev), dput(d["s2"], dev)
    packed = w4.prepack_weights(w13, s13) + w4.prepack_weights(w2, s2)
    t = lambda v: None if v is None else torch.tensor([v], dtype=torch.float32, device=dev)
    out = w4.fused_moe(bf16_dev(d["hidden"], dev), dput(d["topk_ids"], dev), dput(d["topk_weights"], dev),
                       cfg.expert_begin, cfg.E_local, w13, s13, w2, s2, prepacked=packed,
                       a1_scale=t(a1), a2_scale=t(a2))
    torch.cuda.synchronize()
    ref = oracle.fused_moe_static(d["hidden"], d["topk_ids"], d["topk_weights"], cfg.expert_begin,
                                  cfg.E_local, d["w13"], d["s13"], d["w2"], d["s2"], a1, a2)
    assert_bf16_close(bf16_host(out), ref, "static %s %s" % (shape, which))
