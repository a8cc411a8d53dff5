"""Seeded synthetic inputs for MoE expert-parallel dispatch / combine.

This module only draws inputs. It holds none of the dispatch arithmetic
(no counting, no prefix sums, no placement, no reduction), so both the HIP
path and the CPU oracle can consume the same bytes without sharing any of
the method's code.

Every tensor comes from its own numpy stream,
``default_rng(SeedSequence([seed, stream]))``, so one tensor can be
regenerated without drawing the others:

    stream 0  expert choices (topk_idx)
    stream 1  the "-1" (no selection) mask
    stream 2  router logits that become topk_weights
    stream 3  hidden rows x (bf16)
    stream 4  per-128-column fp32 scales
    stream 5  Zipf rank -> expert permutation and the cold-expert set

Workload shapes follow the MoE layer described in the pages: a token batch
``[T, H]`` of bf16 activations, ``topk_idx [T, K]`` int64 with -1 for "no
selection" and ``topk_weights [T, K]`` fp32 (DeepEP代码解读, section
Dispatch, the get_dispatch_layout / dispatch argument lists), and optional
fp32 scales with one value per 128 hidden columns (same section, the tuple
form of ``x``).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

STREAM_TOPK = 0
STREAM_MASK = 1
STREAM_LOGITS = 2
STREAM_X = 3
STREAM_SCALE = 4
STREAM_ZIPF = 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and routing recipe of one synthetic MoE dispatch workload."""

    name: str
    seed: int
    num_tokens: int          # T
    hidden: int              # H
    num_experts: int         # E
    num_topk: int            # K
    num_ranks: int           # R (virtual ranks; rank r owns a contiguous E/R experts)
    scales: bool             # fp32 scale row of H/128 values per token
    routing: str             # "uniform" or "zipf"
    drop_rate: float = 0.0   # probability that a slot is set to -1
    zipf_s: float = 1.2
    cold_experts: int = 0    # experts with zero routing probability (zipf only)
    expert_fn: str = "identity"   # "identity" or "scale" (row * (1 + e/256), bf16)
    payload: str = "bf16"         # "bf16" or "fp8" (e4m3, one byte per element)
    scale_format: str = "f32"     # "f32" (fp32 per 128 columns) or "ue8m0" (packed exponents)
    ranks_per_node: int = 0       # G for num_tokens_per_rdma_rank (0: not asked for)
    # Receive side ("recv" routing): the batch one rank holds after the
    # dispatch. Tokens are drawn with uniform top-K routing over
    # recv_global_experts experts spread over recv_src_ranks ranks and kept
    # when they pick at least one expert of rank recv_rank; ids are local
    # (0 .. num_experts-1) with -1 for experts of other ranks.
    recv_global_experts: int = 0
    recv_src_ranks: int = 0
    recv_rank: int = 0
    # Low-latency (fixed-rectangle) dispatch: tokens arrive as segments of
    # ll_segment tokens (one per source rank); 0 = not a low-latency workload.
    ll_segment: int = 0

    @property
    def scale_cols(self) -> int:
        return self.hidden // 128 if self.scales else 0

    @property
    def scale_words(self) -> int:
        """32-bit words per scale row: S floats, or ceil(S/4) packed UE8M0 words."""
        if not self.scales:
            return 0
        return self.scale_cols if self.scale_format == "f32" else (self.scale_cols + 3) // 4

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, plus the FP8 and receive-side variants of "dsv3". "dsv3" borrows only the public DeepSeek-V3 MoE dimensions
# (hidden 7168, 256 routed experts, top-8); no weights or data are involved.
WORKLOADS = {
    "tiny": Workload("tiny", seed=1, num_tokens=64, hidden=128, num_experts=16,
                     num_topk=2, num_ranks=8, scales=False, routing="uniform",
                     ranks_per_node=2),
    "small": Workload("small", seed=2, num_tokens=2048, hidden=4096, num_experts=64,
                      num_topk=6, num_ranks=8, scales=False, routing="uniform",
                      drop_rate=0.05),
    "dsv3": Workload("dsv3", seed=3, num_tokens=4096, hidden=7168, num_experts=256,
                     num_topk=8, num_ranks=32, scales=True, routing="uniform",
                     ranks_per_node=8),
    "skew": Workload("skew", seed=4, num_tokens=16384, hidden=7168, num_experts=256,
                     num_topk=8, num_ranks=32, scales=True, routing="zipf",
                     zipf_s=1.2, cold_experts=8, ranks_per_node=8),
    "large": Workload("large", seed=5, num_tokens=65536, hidden=7168, num_experts=256,
                      num_topk=8, num_ranks=64, scales=False, routing="uniform",
                      expert_fn="scale", ranks_per_node=8),
    # what one of the 32 ranks of the DeepSeek-V3-shaped setup receives:
    # 32 x 4096 source tokens, each kept with probability
    # 1 - C(248,8)/C(256,8) = 0.2271 (at least one of the rank's 8 experts),
    # i.e. 29765 tokens and, on average, 32768 local slots
    # the same batch dispatched the low-latency way: 32 source ranks of 128
    # decode tokens, every expert's rectangle sized for the worst case
    # (32 x 128 = 4096 rows), FP8 cast on the way
    "dsv3_ll": Workload("dsv3_ll", seed=3, num_tokens=4096, hidden=7168, num_experts=256,
                        num_topk=8, num_ranks=32, scales=False, routing="uniform",
                        ll_segment=128),
    "dsv3_recv": Workload("dsv3_recv", seed=6, num_tokens=29765, hidden=7168, num_experts=8,
                          num_topk=8, num_ranks=1, scales=True, routing="recv",
                          recv_global_experts=256, recv_src_ranks=32, recv_rank=0),
    # the DeepSeek-V3-shaped batch as DeepEP dispatches it for an FP8 grouped
    # GEMM: e4m3 rows and power-of-two (UE8M0) scales packed 4 per int32
    "dsv3_fp8": Workload("dsv3_fp8", seed=3, num_tokens=4096, hidden=7168, num_experts=256,
                         num_topk=8, num_ranks=32, scales=True, routing="uniform",
                         payload="fp8", scale_format="ue8m0", ranks_per_node=8),
}


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def fp32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the raw
    uint16 bit patterns. Used only to manufacture bf16 inputs; the inputs
    are finite draws, so NaN handling is not needed here."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _uniform_distinct(rng: np.random.Generator, T: int, E: int, K: int) -> np.ndarray:
    """K distinct experts per token, uniformly without replacement, in random
    slot order (the first K entries of a uniformly random permutation)."""
    out = np.empty((T, K), dtype=np.int64)
    chunk = max(1, (1 << 22) // max(E, 1))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        keys = rng.random((t1 - t0, E))
        if K < E:
            part = np.argpartition(keys, K, axis=1)[:, :K]
            # argpartition leaves the K smallest keys unordered: order them
            # by key so the slot order is the permutation order.
            sub = np.take_along_axis(keys, part, axis=1)
            order = np.argsort(sub, axis=1, kind="stable")
            out[t0:t1] = np.take_along_axis(part, order, axis=1)
        else:
            out[t0:t1] = np.argsort(keys, axis=1, kind="stable")[:, :K]
    return out


def _zipf_without_replacement(w: Workload) -> np.ndarray:
    """Per token, K experts drawn without replacement with P(rank r) ~ r^-s
    over the warm experts (successive draws renormalised). Implemented with
    Efraimidis-Spirakis keys log(U)/weight: sorting the keys in descending
    order yields a sample with exactly that sequential-draw distribution,
    and the slot order is the draw order. A seeded set of cold experts gets
    weight 0 so that some experts receive no tokens."""
    T, E, K = w.num_tokens, w.num_experts, w.num_topk
    warm = E - w.cold_experts
    if K > warm:
        raise ValueError("top-k larger than the number of warm experts")
    perm = _rng(w.seed, STREAM_ZIPF).permutation(E)      # rank r+1 -> perm[r]
    weight = np.arange(1, warm + 1, dtype=np.float64) ** (-w.zipf_s)
    rng = _rng(w.seed, STREAM_TOPK)
    out = np.empty((T, K), dtype=np.int64)
    chunk = max(1, (1 << 22) // warm)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        u = rng.random((t1 - t0, warm))
        u = np.maximum(u, np.finfo(np.float64).tiny)
        keys = np.log(u) / weight                          # larger key = drawn earlier
        order = np.argsort(-keys, axis=1, kind="stable")[:, :K]
        out[t0:t1] = perm[order]
    return out


def cold_experts(w: Workload) -> np.ndarray:
    """The experts that the zipf recipe never selects (empty for uniform)."""
    if w.routing != "zipf" or w.cold_experts == 0:
        return np.empty(0, dtype=np.int64)
    perm = _rng(w.seed, STREAM_ZIPF).permutation(w.num_experts)
    return np.sort(perm[w.num_experts - w.cold_experts:])


def _received_global(w: Workload) -> np.ndarray:
    """Global top-K rows [T, K] of the tokens rank recv_rank receives: uniform
    routing over recv_global_experts experts, keeping the rows that pick at
    least one of the rank's experts, in draw order, until T are kept."""
    El, lo = w.num_experts, w.recv_rank * w.num_experts
    rng = _rng(w.seed, STREAM_TOPK)
    kept, have = [], 0
    while have < w.num_tokens:
        g = _uniform_distinct(rng, 1 << 14, w.recv_global_experts, w.num_topk)
        g = g[((g >= lo) & (g < lo + El)).any(axis=1)]
        kept.append(g)
        have += len(g)
    return np.concatenate(kept)[:w.num_tokens]


def make_topk(w: Workload) -> np.ndarray:
    """topk_idx [T, K] int64, -1 = no selection."""
    if w.routing == "recv":
        g = _received_global(w)
        lo = w.recv_rank * w.num_experts
        mine = (g >= lo) & (g < lo + w.num_experts)
        return np.ascontiguousarray(np.where(mine, g - lo, -1))
    if w.routing == "uniform":
        topk = _uniform_distinct(_rng(w.seed, STREAM_TOPK), w.num_tokens,
                                 w.num_experts, w.num_topk)
    elif w.routing == "zipf":
        topk = _zipf_without_replacement(w)
    else:
        raise ValueError(f"unknown routing {w.routing!r}")
    if w.drop_rate > 0.0:
        drop = _rng(w.seed, STREAM_MASK).random(topk.shape) < w.drop_rate
        topk[drop] = -1
    return np.ascontiguousarray(topk)


def make_weights(w: Workload, topk: np.ndarray) -> np.ndarray:
    """topk_weights [T, K] fp32: softmax of N(0,1) logits over the token's
    valid slots, 0 on -1 slots, so the valid weights of a token sum to 1."""
    logits = _rng(w.seed, STREAM_LOGITS).standard_normal(topk.shape)
    if w.routing == "recv":
        # the sender's weights: softmax over all K slots of the global row
        # (every slot is valid there); slots of other ranks arrive as 0
        ex = np.exp(logits - logits.max(axis=1, keepdims=True))
        wt = ex / ex.sum(axis=1, keepdims=True)
        return np.ascontiguousarray(np.where(topk >= 0, wt, 0.0).astype(np.float32))
    valid = topk >= 0
    masked = np.where(valid, logits, -np.inf)
    mx = masked.max(axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    ex = np.where(valid, np.exp(masked - mx), 0.0)
    den = ex.sum(axis=1, keepdims=True)
    den = np.where(den > 0.0, den, 1.0)
    return np.ascontiguousarray((ex / den).astype(np.float32))


def make_x(w: Workload, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Hidden rows x [T, H] as raw bf16 bits (uint16), from N(0,1) fp32 draws
    rounded to nearest-even. Drawn in row chunks so the full Large batch
    never needs an fp32 copy at once. ``rows`` selects a subset of tokens
    (the full batch is still drawn in order so the bytes are identical)."""
    T, H = w.num_tokens, w.hidden
    rng = _rng(w.seed, STREAM_X)
    chunk = max(1, (1 << 24) // max(H, 1))
    if rows is None:
        out = np.empty((T, H), dtype=np.uint16)
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            out[t0:t1] = fp32_to_bf16_bits(rng.standard_normal((t1 - t0, H), dtype=np.float32))
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H), dtype=np.uint16)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        sel = np.nonzero((rows >= t0) & (rows < t1))[0]
        block = rng.standard_normal((t1 - t0, H), dtype=np.float32)
        if sel.size:
            out[sel] = fp32_to_bf16_bits(block[rows[sel] - t0])
    return out


def make_scales(w: Workload) -> Optional[np.ndarray]:
    """x_scale [T, H/128] fp32 drawn U(0.01, 1), or None without scales."""
    if not w.scales:
        return None
    s = _rng(w.seed, STREAM_SCALE).uniform(0.01, 1.0, (w.num_tokens, w.scale_cols))
    return np.ascontiguousarray(s.astype(np.float32))


def make_x_fp8(w: Workload) -> np.ndarray:
    """Hidden rows [T, H] as FP8 e4m3 bytes (uint8): the same N(0,1) fp32
    draws as make_x, rounded to e4m3 by torch's float8_e4m3fn conversion."""
    import torch

    T, H = w.num_tokens, w.hidden
    rng = _rng(w.seed, STREAM_X)
    out = np.empty((T, H), dtype=np.uint8)
    chunk = max(1, (1 << 24) // max(H, 1))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        f = torch.from_numpy(rng.standard_normal((t1 - t0, H), dtype=np.float32))
        out[t0:t1] = f.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out


def make_scales_ue8m0(w: Workload) -> Optional[np.ndarray]:
    """Per-128-column power-of-two scales as UE8M0 exponent bytes (2^k with
    k uniform in [-10, 2], byte = 127 + k), packed four per little-endian
    uint32 word: [T, ceil(S/4)]; bytes past S in the last word are 0."""
    if not w.scales:
        return None
    S, W = w.scale_cols, w.scale_words
    k = _rng(w.seed, STREAM_SCALE).integers(-10, 3, size=(w.num_tokens, S))
    b = np.zeros((w.num_tokens, 4 * W), dtype=np.uint8)
    b[:, :S] = (127 + k).astype(np.uint8)
    return np.ascontiguousarray(b).view("<u4").reshape(w.num_tokens, W).astype(np.uint32)


def make_inputs(w: Workload, with_x: bool = True) -> dict:
    """All inputs of one workload as host numpy arrays."""
    topk = make_topk(w)
    fp8 = w.payload == "fp8"
    if fp8:
        x = make_x_fp8(w) if with_x else None
        xs = make_scales_ue8m0(w) if w.scale_format == "ue8m0" else make_scales(w)
    else:
        x = make_x(w) if with_x else None
        xs = make_scales(w)
    return {"topk_idx": topk, "topk_weights": make_weights(w, topk), "x": x, "x_scale": xs}


def get(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise ValueError(f"unknown workload {name!r}; choose from {sorted(WORKLOADS)}") from None
