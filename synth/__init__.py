"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module holds no arithmetic of the scoring method.  It only draws numbers:

* ``u64(seed, stream, index)`` is SplitMix64 used as a counter-based generator:
  the key ``mix64(seed * GAMMA + stream * STREAM_MUL)`` is the generator state,
  and output ``i`` is ``mix64(key + (i + 1) * GAMMA)``, i.e. the (i+1)-th output
  of the published SplitMix64 sequence started at that key (Steele, Lea and
  Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014).
* ``normals`` turns pairs of outputs into N(0, 1) draws by the Box-Muller
  transform (u1 in (0, 1], u2 in [0, 1), 53-bit mantissas), element ``2p`` is the
  cosine branch and ``2p + 1`` the sine branch of pair ``p``.
* ``to_bf16`` rounds float32 to bfloat16 bits with round-to-nearest-even.

Streams: 1 = queries, 2 = keys, 3 = planted directions, 4 = span positions,
5 = score arrays for selection tests.  Tensors are returned as bfloat16 bit
patterns (``uint16``) or float32, in the layouts the library consumes:
Q ``[H_q][W][d_k]`` and K ``[H_kv][L][d_k]`` (KV-head-major).

The workloads mirror the shapes of the models the pages study (Llama-3.1-8B and
Mistral-7B GQA layers: 32 query heads, 8 KV heads, head dim 128) at 16K-128K
context, with planted high-similarity key spans standing in for the
needle/retrieval structure of the pages' long-context benchmarks.  No item of
any benchmark is reproduced.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
STREAM_MUL = 0xD1B54A32D192ED03
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
_M64 = (1 << 64) - 1

STREAM_Q, STREAM_K, STREAM_DIR, STREAM_SPAN, STREAM_SCORES = 1, 2, 3, 4, 5


def _mix64_scalar(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * MIX1) & _M64
    z = ((z ^ (z >> 27)) * MIX2) & _M64
    return z ^ (z >> 31)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(MIX1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(MIX2)
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> int:
    return _mix64_scalar(seed * GAMMA + stream * STREAM_MUL)


def u64(seed: int, stream: int, index) -> np.ndarray:
    """Counter-based SplitMix64 output(s) for integer index/indices >= 0."""
    key = np.uint64(stream_key(seed, stream))
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(key + (idx + np.uint64(1)) * np.uint64(GAMMA))


def uniform_int(seed: int, stream: int, index: int, n: int) -> int:
    """Integer in [0, n) from one generator output (modulo reduction)."""
    return int(u64(seed, stream, index)) % n


def normals(seed: int, stream: int, offset: int, count: int) -> np.ndarray:
    """N(0,1) float64 draws number offset .. offset+count-1 of (seed, stream)."""
    if count <= 0:
        return np.zeros(0, dtype=np.float64)
    p0 = offset // 2
    p1 = (offset + count - 1) // 2
    pairs = np.arange(p0, p1 + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x1 = u64(seed, stream, pairs * np.uint64(2))
        x2 = u64(seed, stream, pairs * np.uint64(2) + np.uint64(1))
    u1 = ((x1 >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)
    u2 = (x2 >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    r = np.sqrt(-2.0 * np.log(u1))
    th = 2.0 * math.pi * u2
    out = np.empty(2 * len(pairs), dtype=np.float64)
    out[0::2] = r * np.cos(th)
    out[1::2] = r * np.sin(th)
    s = offset - 2 * p0
    return out[s:s + count]


def to_bf16(x) -> np.ndarray:
    """float -> float32 (RNE) -> bfloat16 bits (RNE), as uint16."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def unit_direction(seed: int, index: int, d_k: int) -> np.ndarray:
    v = normals(seed, STREAM_DIR, index * d_k, d_k)
    return v / np.linalg.norm(v)


# ---------------------------------------------------------------------------
# Workload descriptors
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Layer:
    """One layer's scoring inputs plus the planted ground truth."""
    Q: np.ndarray            # uint16 bf16 bits [H_q][W][d_k]
    K: np.ndarray            # uint16 bf16 bits [H_kv][L][d_k]
    L: int
    W: int
    d_k: int
    H_q: int
    H_kv: int
    q_pos0: int
    spans: List[Tuple[int, int]]   # [start, end) token ranges planted in every KV head

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv


def beta_for(d_k: int, lift: float) -> float:
    """Amplitude whose square over sqrt(d_k) equals the wanted logit lift."""
    return math.sqrt(lift * math.sqrt(d_k))


def gaussian_layer(seed: int, L: int, W: int, d_k: int, H_q: int, H_kv: int,
                   q_pos0: Optional[int] = None, n_spans: int = 0, span_len: int = 0,
                   lift: float = 2.0, span_region: Optional[int] = None,
                   fixed_span_seed: Optional[int] = None, n_fixed: int = 0,
                   dir_seed: Optional[int] = None) -> Layer:
    """N(0,1) bf16 Q/K; optional planted spans sharing a direction with the window.

    Planted keys of KV head g and all W window rows of its G query heads get
    ``+beta * u_g`` (unit direction u_g), which lifts their logit by ``lift``.
    Spans lie in the candidate prefix [0, span_region) (default L - W).  With
    ``n_fixed > 0`` the first n_fixed span slots are drawn from
    ``fixed_span_seed`` (identical across layers) and the rest from ``seed``.
    """
    if q_pos0 is None:
        q_pos0 = L - W
    G = H_q // H_kv
    beta = beta_for(d_k, lift)
    dseed = seed if dir_seed is None else dir_seed
    spans: List[Tuple[int, int]] = []
    if n_spans:
        region = (L - W) if span_region is None else span_region
        seg = region // n_spans
        starts = []
        for i in range(n_spans):
            s_seed = fixed_span_seed if (i < n_fixed and fixed_span_seed is not None) else seed
            room = seg - span_len + 1
            starts.append(i * seg + uniform_int(s_seed, STREAM_SPAN, i, room))
        spans = [(s, s + span_len) for s in starts]
    dirs = [unit_direction(dseed, g, d_k) for g in range(H_kv)] if n_spans else None

    K = np.empty((H_kv, L, d_k), dtype=np.uint16)
    for g in range(H_kv):
        kf = normals(seed, STREAM_K, g * L * d_k, L * d_k).reshape(L, d_k)
        if n_spans:
            for (a, b) in spans:
                kf[a:b] += beta * dirs[g]
        K[g] = to_bf16(kf.astype(np.float32))
    qf = normals(seed, STREAM_Q, 0, H_q * W * d_k).reshape(H_q, W, d_k)
    if n_spans:
        for h in range(H_q):
            qf[h] += beta * dirs[h // G]
    Q = to_bf16(qf.astype(np.float32))
    return Layer(Q=Q, K=K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0, spans=spans)


def plant_outliers(ly: Layer, seed: int, outliers, a: float = 16.0) -> Layer:
    """Plant outlier keys: a few logits far above every other logit of some rows.

    ``outliers`` lists ``(g, head_slot, t, lift)``: query head ``g * G +
    head_slot``'s window rows get ``+a * u`` and key ``t`` of KV head ``g`` gets
    ``+(lift * sqrt(d_k) / a) * u``, with ``u`` a unit direction drawn for that
    (g, head_slot) pair, so the planted logit ``q . k / sqrt(d_k)`` sits about
    ``lift`` above the row's ordinary logits (attention sinks and outlier keys of
    real models).  The rows of one head share one direction, whatever lifts its
    outliers carry; each row is lifted once.  Returns a new Layer; ``ly`` is
    unchanged.
    """
    G = ly.H_q // ly.H_kv
    q = bf16_to_f32(ly.Q).astype(np.float64)
    k = bf16_to_f32(ly.K).astype(np.float64)
    lifted = set()
    for (g, hs, t, lift) in outliers:
        u = unit_direction(seed, 1000 + g * G + hs, ly.d_k)
        if (g, hs) not in lifted:
            q[g * G + hs] += a * u
            lifted.add((g, hs))
        k[g, t] += (lift * math.sqrt(ly.d_k) / a) * u
    return dataclasses.replace(ly, Q=to_bf16(q.astype(np.float32)), K=to_bf16(k.astype(np.float32)))


def tiny(seed: int = 0) -> Layer:
    """1 layer, H_q=4, H_kv=1, d_k=64, L=512, W=16, N(0,1) bf16."""
    return gaussian_layer(seed, L=512, W=16, d_k=64, H_q=4, H_kv=1)


def llama_layer(L: int = 32768, seed: int = 1, n_spans: int = 8, span_len: int = 256) -> Layer:
    """Llama-3.1-8B-shaped layer (32/8 heads, d_k 128, W 32) with planted spans."""
    return gaussian_layer(seed, L=L, W=32, d_k=128, H_q=32, H_kv=8,
                          n_spans=n_spans, span_len=span_len, lift=2.0)


def mistral_layer(L: int = 131072, seed: int = 2, n_spans: int = 16, span_len: int = 512) -> Layer:
    """Mistral-7B-shaped layer at long context (32/8 heads, d_k 128, W 32)."""
    return gaussian_layer(seed, L=L, W=32, d_k=128, H_q=32, H_kv=8,
                          n_spans=n_spans, span_len=span_len, lift=2.0)


def cross_layer(layer: int, L: int = 16384, base_seed: int = 3, H_q: int = 32, H_kv: int = 8,
                n_spans: int = 8, span_len: int = 256) -> Layer:
    """Layer ``layer`` of the cross-layer workload: slots 0-3 fixed, 4-7 per layer."""
    return gaussian_layer(base_seed + layer, L=L, W=32, d_k=128, H_q=H_q, H_kv=H_kv,
                          n_spans=n_spans, span_len=span_len, lift=2.0,
                          fixed_span_seed=base_seed, n_fixed=4)


def last_token_layer(L: int = 131072, seed: int = 5, n_spans: int = 16, span_len: int = 512) -> Layer:
    """Mistral-7B-shaped layer with one query row, the last prompt token (GemFilter)."""
    return gaussian_layer(seed, L=L, W=1, d_k=128, H_q=32, H_kv=8, q_pos0=L - 1,
                          n_spans=n_spans, span_len=span_len, lift=2.0, span_region=L - 1)


def lookahead_layer(layer: int = 0, L: int = 131072, k: int = 8, base_seed: int = 6,
                    n_spans: int = 16, span_len: int = 512) -> Layer:
    """Layer ``layer`` of a Mistral-7B-shaped model with k lookahead queries after the
    prompt (Speculative Prefill); span slots 0-7 fixed across layers."""
    return gaussian_layer(base_seed + layer, L=L, W=k, d_k=128, H_q=32, H_kv=8, q_pos0=L,
                          n_spans=n_spans, span_len=span_len, lift=2.0, span_region=L,
                          fixed_span_seed=base_seed, n_fixed=n_spans // 2)


@dataclasses.dataclass
class Chunk:
    """Chunked-prefill block-selection inputs."""
    Qc: np.ndarray   # uint16 [H_q][Lq][d_k]
    K: np.ndarray    # uint16 [H_kv][L][d_k]
    L: int
    Lq: int
    d_k: int
    H_q: int
    H_kv: int
    q_pos0: int
    block: int
    spans: List[List[Tuple[int, int]]]   # per KV head


def chunk_select(L: int = 131072, Lq: int = 1024, seed: int = 4, H_q: int = 32, H_kv: int = 8,
                 d_k: int = 128, block: int = 64, n_spans: int = 16, span_len: int = 512,
                 lift: float = 10.0) -> Chunk:
    """Chunk of Lq queries at the end of an L-token KV cache, with per-head planted spans.

    For KV head g, span s uses direction v[h, rho] with h = g*G + (s mod G) and
    rho = (s div G) mod 4; rows of query block i of head h get +gamma*v[h, i mod 4],
    so each (head, query block) pair matches one span.
    """
    G = H_q // H_kv
    q_pos0 = L - Lq
    gamma = beta_for(d_k, lift)
    seg = q_pos0 // n_spans
    dirs = {(h, r): unit_direction(seed, h * 4 + r, d_k) for h in range(H_q) for r in range(4)}
    K = np.empty((H_kv, L, d_k), dtype=np.uint16)
    spans_all = []
    for g in range(H_kv):
        kf = normals(seed, STREAM_K, g * L * d_k, L * d_k).reshape(L, d_k)
        spans = []
        for s in range(n_spans):
            a = s * seg + uniform_int(seed, STREAM_SPAN, g * n_spans + s, seg - span_len + 1)
            h = g * G + (s % G)
            rho = (s // G) % 4
            kf[a:a + span_len] += gamma * dirs[(h, rho)]
            spans.append((a, a + span_len))
        spans_all.append(spans)
        K[g] = to_bf16(kf.astype(np.float32))
    qf = normals(seed, STREAM_Q, 0, H_q * Lq * d_k).reshape(H_q, Lq, d_k)
    for h in range(H_q):
        for i in range(Lq // block):
            qf[h, i * block:(i + 1) * block] += gamma * dirs[(h, i % 4)]
    Qc = to_bf16(qf.astype(np.float32))
    return Chunk(Qc=Qc, K=K, L=L, Lq=Lq, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0,
                 block=block, spans=spans_all)


# ---------------------------------------------------------------------------
# Score arrays for selection tests (float32, with forced ties)
# ---------------------------------------------------------------------------

def score_array(seed: int, H: int, n: int, levels: int = 0, signed: bool = False,
                with_zeros: bool = False) -> np.ndarray:
    """float32 [H][n]; ``levels > 0`` quantises to that many values to force ties.

    With ``with_zeros`` a fifth of the entries are set to +0.0 or -0.0.
    """
    x = normals(seed, STREAM_SCORES, 0, H * n).reshape(H, n)
    if not signed:
        x = np.exp(x)          # positive, heavy right tail like attention mass
    if levels > 0:
        lo, hi = x.min(), x.max()
        x = np.round((x - lo) / (hi - lo + 1e-30) * (levels - 1)) / max(levels - 1, 1)
        if signed:
            x = x - 0.5
    x = x.astype(np.float32)
    if with_zeros:
        sel = (u64(seed, STREAM_SCORES + 100, np.arange(H * n)) % np.uint64(5)) == 0
        neg = (u64(seed, STREAM_SCORES + 200, np.arange(H * n)) % np.uint64(2)) == 0
        flat = x.reshape(-1)
        flat[sel & neg] = np.float32(-0.0)
        flat[sel & ~neg] = np.float32(0.0)
    return x


def priority_array(seed: int, H: int, n: int, frac_num: int = 1, frac_den: int = 10) -> np.ndarray:
    """uint8 [H][n] with about frac_num/frac_den ones."""
    r = u64(seed, STREAM_SCORES + 300, np.arange(H * n)) % np.uint64(frac_den)
    return (r < np.uint64(frac_num)).astype(np.uint8).reshape(H, n)


def block_mask(seed: int, H_q: int, n_qb: int, n_kvb: int, density_den: int = 8) -> np.ndarray:
    """uint8 [H_q][n_qb][n_kvb] with about 1/density_den ones."""
    r = u64(seed, STREAM_SCORES + 400, np.arange(H_q * n_qb * n_kvb)) % np.uint64(density_den)
    return (r == 0).astype(np.uint8).reshape(H_q, n_qb, n_kvb)
