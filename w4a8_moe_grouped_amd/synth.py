"""Seeded synthetic inputs for the W4AFP8 fused-MoE forward.

This module only draws inputs; it holds none of the method's arithmetic
(no quantisation, no GEMM, no activation, no combine).  Both the HIP path's
tests and benchmark and the CPU oracle take their inputs from here, so that
the two sides see byte-identical data.

Random numbers come from one counter-based generator (SplitMix64, the
finaliser published by Steele, Lea and Flood, 2014): element ``i`` of stream
``s`` under ``seed`` is ``mix64((seed ^ s*G) + (i+1)*G)`` with
``G = 0x9E3779B97F4A7C15`` and all arithmetic mod 2**64.  Streams: 1 router
logits, 2 activations, 3 outlier mask, 4 w13 bytes, 5 w13 scales, 6 w2
bytes, 7 w2 scales, 8 the expert-popularity permutation.

Recipes (the workloads the pages describe, at the sizes of the five
benchmark configurations):
  * activations: N(0, 1) by Box-Muller from two uniforms, rounded to bf16;
    the dense case multiplies an entry by 20 with probability 0.01;
  * int4 weights: uniform random bytes (each nibble uniform on -8..7);
  * weight scales: fp32 uniform on [0.002, 0.02];
  * fp4 weights (the FP4 E2M1 variant): uniform random bytes (each nibble
    uniform over the 16 e2m1 codes), one UE8M0 scale byte per 32 K drawn
    uniformly from 2^-9 .. 2^-6 (streams 5 and 7, top two bits of a draw);
  * routing: N(0, 1) logits over all experts (plus a Zipf(s) popularity bias
    -s*ln(rank) for the skewed cases), softmax in fp64, top-k with ties to
    the lower expert id, weights renormalised over the top-k, stored fp32.
    Only experts [expert_begin, expert_begin + E_local) are this GPU's share.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 21
_WORKERS = max(1, min(16, os.cpu_count() or 1))

STREAM_LOGITS, STREAM_X, STREAM_OUTLIER, STREAM_W13, STREAM_S13, STREAM_W2, STREAM_S2, \
    STREAM_PERM = 1, 2, 3, 4, 5, 6, 7, 8


# ---- the counter-based generator ---------------------------------------------

def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def draw_u64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Elements [start, start+count) of one stream, as uint64."""
    with np.errstate(over="ignore"):
        base = np.uint64(seed) ^ (np.uint64(stream) * GOLDEN)
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        return _mix64(base + i * GOLDEN)


def draw_uniform(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Uniform doubles in [0, 1) from the top 53 bits."""
    u = draw_u64(seed, stream, start, count) >> np.uint64(11)
    return u.astype(np.float64) * (1.0 / 9007199254740992.0)


def _parallel_chunks(total: int, fn) -> None:
    """Run fn(c0, c1) over [0, total) in chunks; numpy releases the GIL inside
    its ufuncs, so threads overlap.  Each chunk depends only on its own counter
    range, so the result does not depend on the scheduling."""
    spans = [(c0, min(total, c0 + _CHUNK)) for c0 in range(0, total, _CHUNK)]
    if len(spans) <= 1:
        for c0, c1 in spans:
            fn(c0, c1)
        return
    with concurrent.futures.ThreadPoolExecutor(max_workers=_WORKERS) as ex:
        for _ in ex.map(lambda sp: fn(*sp), spans):
            pass


def draw_normal(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """N(0, 1) doubles; normal i uses uniforms 2i and 2i+1 (Box-Muller, cos branch)."""
    out = np.empty(count, np.float64)

    def fill(c0, c1):
        u = draw_uniform(seed, stream, 2 * (start + c0), 2 * (c1 - c0))
        u1, u2 = u[0::2], u[1::2]
        out[c0:c1] = np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * np.pi * u2)

    _parallel_chunks(count, fill)
    return out


def draw_bytes(seed: int, stream: int, count: int) -> np.ndarray:
    """Uniform random bytes: byte b of draw i is element 8i+b (little endian)."""
    n64 = (count + 7) // 8
    out = np.empty(n64 * 8, np.uint8)

    def fill(c0, c1):
        out[8 * c0:8 * c1] = draw_u64(seed, stream, c0, c1 - c0).view(np.uint8)

    _parallel_chunks(n64, fill)
    return out[:count]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---- configurations ------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    I: int
    E_total: int
    topk: int
    expert_begin: int
    E_local: int
    routing: str = "uniform"  # "uniform" | "zipf_perm" | "zipf_id"
    zipf_s: float = 1.2
    seed: int = 0
    desc: str = ""


@dataclasses.dataclass(frozen=True)
class DenseConfig:
    name: str
    M: int
    K: int
    N: int
    outlier_p: float = 0.01
    outlier_mult: float = 20.0
    seed: int = 0
    desc: str = ""


CONFIGS: Dict[str, object] = {
    "tiny": MoEConfig("tiny", T=16, H=256, I=128, E_total=4, topk=2, expert_begin=0, E_local=4,
                      desc="tiny fused MoE, T=16 H=256 I=128 E=4 top-2"),
    "dense": DenseConfig("dense", M=128, K=7168, N=2048,
                         desc="dense W4AFP8 linear M=128 K=7168 N=2048, 1% x20 outliers"),
    "decode": MoEConfig("decode", T=64, H=7168, I=2048, E_total=256, topk=8, expert_begin=0,
                        E_local=32, desc="decode T=64, experts 0..31 of 256, top-8"),
    "prefill": MoEConfig("prefill", T=4096, H=7168, I=2048, E_total=256, topk=8, expert_begin=0,
                         E_local=32, desc="prefill T=4096, experts 0..31 of 256, top-8"),
    "prefill_ep8": MoEConfig("prefill_ep8", T=32768, H=7168, I=2048, E_total=256, topk=8,
                             expert_begin=0, E_local=32,
                             desc="prefill EP8 rank share: 8x4096 tokens, ~1024 pairs/expert"),
    "skew_perm": MoEConfig("skew_perm", T=256, H=7168, I=2048, E_total=256, topk=8,
                           expert_begin=0, E_local=32, routing="zipf_perm",
                           desc="Zipf(1.2) popularity, rank = seeded permutation"),
    "skew_id": MoEConfig("skew_id", T=256, H=7168, I=2048, E_total=256, topk=8,
                         expert_begin=0, E_local=32, routing="zipf_id",
                         desc="Zipf(1.2) popularity, rank = expert id + 1"),
}


# ---- MoE inputs ------------------------------------------------------------------

def gen_hidden(cfg: MoEConfig, t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
    """bf16 bits [t1-t0, H] of tokens t0..t1-1 (stream 2, element t*H + h)."""
    t1 = cfg.T if t1 is None else t1
    n = (t1 - t0) * cfg.H
    out = np.empty(n, np.uint16)

    def fill(c0, c1):
        out[c0:c1] = to_bf16_bits(draw_normal(cfg.seed, STREAM_X, t0 * cfg.H + c0, c1 - c0))

    _parallel_chunks(n, fill)
    return out.reshape(t1 - t0, cfg.H)


def popularity_ranks(cfg: MoEConfig) -> np.ndarray:
    """Rank r_e >= 1 of each expert for the Zipf bias."""
    E = cfg.E_total
    if cfg.routing == "zipf_id":
        return np.arange(1, E + 1, dtype=np.float64)
    # Fisher-Yates over 0..E-1 driven by stream 8
    perm = np.arange(E)
    u = draw_uniform(cfg.seed, STREAM_PERM, 0, E)
    for i in range(E - 1, 0, -1):
        j = int(u[E - 1 - i] * (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return (perm + 1).astype(np.float64)


def gen_routing(cfg: MoEConfig, t0: int = 0, t1: Optional[int] = None):
    """(topk_ids int32 [n, k] of global expert ids, topk_weights fp32 [n, k])."""
    t1 = cfg.T if t1 is None else t1
    n, E, k = t1 - t0, cfg.E_total, cfg.topk
    logits = draw_normal(cfg.seed, STREAM_LOGITS, t0 * E, n * E).reshape(n, E)
    if cfg.routing in ("zipf_perm", "zipf_id"):
        logits = logits - cfg.zipf_s * np.log(popularity_ranks(cfg))[None, :]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p = p / p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]  # ties -> lower id
    top = np.take_along_axis(p, order, axis=1)
    w = top / top.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def gen_expert_weights(cfg: MoEConfig, seed: Optional[int] = None):
    """(w13 [E_l, 2I, H/2] u8, s13 [E_l, 2I, H/128] f32, w2 [E_l, H, I/2] u8,
    s2 [E_l, H, I/128] f32) for the local experts."""
    seed = cfg.seed if seed is None else seed
    E, H, I = cfg.E_local, cfg.H, cfg.I
    w13 = draw_bytes(seed, STREAM_W13, E * 2 * I * H // 2).reshape(E, 2 * I, H // 2)
    s13 = (0.002 + 0.018 * draw_uniform(seed, STREAM_S13, 0, E * 2 * I * (H // 128))) \
        .astype(np.float32).reshape(E, 2 * I, H // 128)
    w2 = draw_bytes(seed, STREAM_W2, E * H * I // 2).reshape(E, H, I // 2)
    s2 = (0.002 + 0.018 * draw_uniform(seed, STREAM_S2, 0, E * H * (I // 128))) \
        .astype(np.float32).reshape(E, H, I // 128)
    return w13, s13, w2, s2


def gen_expert_weights_fp4(cfg: MoEConfig, seed: Optional[int] = None):
    """(w13 [E_l, 2I, H/2] u8 e2m1 nibbles, s13 [E_l, 2I, H/32] u8 UE8M0,
    w2 [E_l, H, I/2] u8, s2 [E_l, H, I/32] u8) for the local experts."""
    seed = cfg.seed if seed is None else seed
    E, H, I = cfg.E_local, cfg.H, cfg.I
    w13 = draw_bytes(seed, STREAM_W13, E * 2 * I * H // 2).reshape(E, 2 * I, H // 2)
    w2 = draw_bytes(seed, STREAM_W2, E * H * I // 2).reshape(E, H, I // 2)
    ue = lambda stream, n: (118 + (draw_u64(seed, stream, 0, n) >> np.uint64(62))).astype(np.uint8)
    s13 = ue(STREAM_S13, E * 2 * I * (H // 32)).reshape(E, 2 * I, H // 32)
    s2 = ue(STREAM_S2, E * H * (I // 32)).reshape(E, H, I // 32)
    return w13, s13, w2, s2


def gen_moe_fp4(cfg: MoEConfig, seed: Optional[int] = None) -> dict:
    ids, w = gen_routing(cfg)
    w13, s13, w2, s2 = gen_expert_weights_fp4(cfg, seed)
    return dict(hidden=gen_hidden(cfg), topk_ids=ids, topk_weights=w,
                w13=w13, s13=s13, w2=w2, s2=s2)


def gen_moe(cfg: MoEConfig, seed: Optional[int] = None) -> dict:
    ids, w = gen_routing(cfg)
    w13, s13, w2, s2 = gen_expert_weights(cfg, seed)
    return dict(hidden=gen_hidden(cfg), topk_ids=ids, topk_weights=w,
                w13=w13, s13=s13, w2=w2, s2=s2)


def routing_stats(cfg: MoEConfig, topk_ids: np.ndarray) -> dict:
    """Local pair count P, active local experts A and the per-expert histogram."""
    loc = topk_ids.ravel().astype(np.int64) - cfg.expert_begin
    loc = loc[(loc >= 0) & (loc < cfg.E_local)]
    hist = np.bincount(loc, minlength=cfg.E_local)
    return dict(P=int(loc.size), A=int(np.count_nonzero(hist)), hist=hist)


# ---- dense inputs ------------------------------------------------------------------

def gen_dense(cfg: DenseConfig, seed: Optional[int] = None):
    """(x bf16 bits [M, K], w u8 [N, K/2], sw f32 [N, K/128])."""
    seed = cfg.seed if seed is None else seed
    M, K, N = cfg.M, cfg.K, cfg.N
    z = draw_normal(seed, STREAM_X, 0, M * K)
    hit = draw_uniform(seed, STREAM_OUTLIER, 0, M * K) < cfg.outlier_p
    z = np.where(hit, z * cfg.outlier_mult, z)
    x = to_bf16_bits(z).reshape(M, K)
    w = draw_bytes(seed, STREAM_W13, N * K // 2).reshape(N, K // 2)
    sw = (0.002 + 0.018 * draw_uniform(seed, STREAM_S13, 0, N * (K // 128))) \
        .astype(np.float32).reshape(N, K // 128)
    return x, w, sw


def random_moe(T: int, H: int, I: int, E_total: int, topk: int, expert_begin: int,
               E_local: int, seed: int, routing: str = "uniform") -> tuple:
    """An ad-hoc configuration plus its inputs (for edge-case tests)."""
    cfg = MoEConfig("adhoc", T=T, H=H, I=I, E_total=E_total, topk=topk,
                    expert_begin=expert_begin, E_local=E_local, routing=routing, seed=seed)
    return cfg, gen_moe(cfg)


def random_moe_fp4(T: int, H: int, I: int, E_total: int, topk: int, expert_begin: int,
                   E_local: int, seed: int, routing: str = "uniform") -> tuple:
    """As random_moe, with fp4 e2m1 weights and UE8M0 per-32 scales."""
    cfg = MoEConfig("adhoc", T=T, H=H, I=I, E_total=E_total, topk=topk,
                    expert_begin=expert_begin, E_local=E_local, routing=routing, seed=seed)
    return cfg, gen_moe_fp4(cfg)
