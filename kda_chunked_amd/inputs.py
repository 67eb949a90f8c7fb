"""Seeded synthetic inputs for the KDA training path.

This module draws random numbers and rounds them to the storage dtypes; it
holds none of the method's arithmetic. Both the GPU path's tests/bench and
the oracle consume the arrays it returns, so the two sides always see the
same bits.

Workloads. The deterministic KDA package's timing rows (flashinfer PR #8909,
timing tables and their row-key paragraph) are named 1doc (one 16384-token
document, 64 heads), 4doc (8192/4096/3072/1024 tokens, 64 heads), R2 (16384
tokens in 3 unequal documents, 4 heads) and m2 (2048/1500 tokens, 4 heads),
with bf16 q/k/v/beta, an fp32 gate and head dim 128. The pages give no value
distributions; the ones below are the recipe this repository fixes:

* q, k, v, dO: standard normal, drawn as float32, rounded to bf16 (RNE).
  With the L2 norm off, q and k are first normalised per (token, head) in
  float32, then rounded once to bf16 (so they are only nearly unit-norm).
  With the fused L2 norm, q and k are raw N(0,1) values.
* beta: sigmoid of a standard normal, rounded to bf16.
* gate form g: logsigmoid(x)/16 of a standard normal x, in float64, stored
  as float32.
* gate form raw: a = bf16(N(0,1)); A_log ~ U(lo, hi) float32 per head;
  dt_bias ~ N(0, 0.5) float32 per (head, channel), 0.5 being the std.
* draw order from numpy.random.default_rng(seed): q, k, v, beta-x, gate-x,
  dO, then A_log and dt_bias for the raw form.

bf16 values are returned as uint16 bit patterns (numpy has no bf16 dtype);
``bf16_to_f32`` widens them exactly.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HEAD_DIM = 128


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    if nan.any():
        out = np.where(nan, np.uint16(0x7FC0), out)
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    doc_lens: tuple
    H: int
    gate: str                 # "g" or "raw"
    l2norm: bool              # fused in-kernel L2 norm on raw q, k
    alog_range: tuple = (0.0, float(np.log(16.0)))
    seed: int = 0
    backward: tuple = ("saved",)
    D: int = HEAD_DIM

    @property
    def T(self) -> int:
        return int(sum(self.doc_lens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.doc_lens)]).astype(np.int32)

    @property
    def key(self) -> str:
        return f"{self.name}:{self.gate}:{'fused' if self.l2norm else 'off'}"


# The five workloads, in order: tiny, m2, R2, 1doc, 4doc fast-decay.
WORKLOADS = [
    Workload("tiny", (200, 56), 2, "g", False, seed=0),
    Workload("m2", (2048, 1500), 4, "g", False, seed=1),
    Workload("R2", (9001, 5120, 2263), 4, "raw", False, (0.0, float(np.log(16.0))), seed=2),
    Workload("1doc", (16384,), 64, "g", True, seed=3),
    Workload("4doc", (8192, 4096, 3072, 1024), 64, "raw", False,
             (float(np.log(4.0)), float(np.log(32.0))), seed=4, backward=("saved", "replay")),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def _normalise_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Draw the inputs of workload ``w``. Returns numpy arrays:
    q, k, v, beta, dO (uint16 bf16 bits), gate (float32 g, or uint16 bf16 a),
    A_log, dt_bias (float32, raw form only), cu_seqlens (int32)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    T, H, D = w.T, w.H, w.D
    q = rng.standard_normal((T, H, D), dtype=np.float32)
    k = rng.standard_normal((T, H, D), dtype=np.float32)
    v = rng.standard_normal((T, H, D), dtype=np.float32)
    bx = rng.standard_normal((T, H), dtype=np.float32)
    gx = rng.standard_normal((T, H, D), dtype=np.float32)
    dO = rng.standard_normal((T, H, D), dtype=np.float32)
    if not w.l2norm:
        q = _normalise_rows(q)
        k = _normalise_rows(k)
    out = {
        "cu_seqlens": w.cu_seqlens,
        "q": f32_to_bf16(q),
        "k": f32_to_bf16(k),
        "v": f32_to_bf16(v),
        "beta": f32_to_bf16((1.0 / (1.0 + np.exp(-bx.astype(np.float64)))).astype(np.float32)),
        "dO": f32_to_bf16(dO),
    }
    if w.gate == "g":
        x = gx.astype(np.float64)
        logsig = np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))
        out["gate"] = (logsig / 16.0).astype(np.float32)
    else:
        out["gate"] = f32_to_bf16(gx)
        lo, hi = w.alog_range
        out["A_log"] = rng.uniform(lo, hi, H).astype(np.float32)
        out["dt_bias"] = rng.normal(0.0, 0.5, (H, D)).astype(np.float32)
    return out


def custom(doc_lens, H, gate="g", l2norm=False, alog_range=(0.0, float(np.log(16.0))),
           seed=0, D=HEAD_DIM, name="custom") -> Workload:
    """A workload of arbitrary document lengths with the same distributions."""
    return Workload(name, tuple(int(x) for x in doc_lens), int(H), gate, bool(l2norm),
                    tuple(alog_range), int(seed), D=int(D))


def as_f64(inp: dict) -> dict:
    """Exact float64 copies of every floating input (for the oracle)."""
    out = {}
    for key in ("q", "k", "v", "beta", "dO"):
        out[key] = bf16_to_f32(inp[key]).astype(np.float64)
    g = inp["gate"]
    out["gate"] = (bf16_to_f32(g) if g.dtype == np.uint16 else g).astype(np.float64)
    for key in ("A_log", "dt_bias"):
        if key in inp:
            out[key] = inp[key].astype(np.float64)
    out["cu_seqlens"] = inp["cu_seqlens"].astype(np.int64)
    return out


# ---------------------------------------------------------------- conv1d + SiLU
#
# The width-4 causal conv1d + SiLU that precedes the state passing in the KDA
# module forward (flashinfer PR #7176, description): x is the packed [T, D]
# projection input (D = q, k and v channels of every head), with the recipe
# x, dy ~ N(0, 1) rounded to bf16; taps w ~ U(-1/2, 1/2) and bias
# b ~ U(-1/2, 1/2) in float32 (the uniform bound 1/sqrt(fan_in) of a width-4
# depthwise conv); halo ~ N(0, 1) bf16, the 3 tokens before x[0] of a
# fragment that continues a document. Draw order: x, dy, w, b, halo.


@dataclass(frozen=True)
class ConvWorkload:
    name: str
    doc_lens: tuple
    D: int
    bias: bool
    halo: bool
    seed: int = 0

    @property
    def T(self) -> int:
        return int(sum(self.doc_lens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.doc_lens)]).astype(np.int32)


CONV_WORKLOADS = [
    ConvWorkload("conv_tiny", (200, 56), 256, True, True, seed=10),
    ConvWorkload("conv_ragged", (2, 0, 1, 70, 3, 0, 64, 130), 512, True, True, seed=11),
    # a channel count that is no multiple of a workgroup's channels (256 or 512):
    # workgroups with idle lanes
    ConvWorkload("conv_narrow", (1, 66, 0, 190), 136, True, True, seed=13),
    # the 4doc layout with the q, k, v channels of 64 heads x 128, as a context
    # fragment that continues its first document (halo on), no bias
    ConvWorkload("conv_4doc", (8192, 4096, 3072, 1024), 3 * 64 * 128, False, True, seed=12),
]
CONV_BY_NAME = {w.name: w for w in CONV_WORKLOADS}


def make_conv_inputs(w: ConvWorkload, seed: int | None = None) -> dict:
    """x, dy, halo (uint16 bf16 bits), w, b (float32), cu_seqlens (int32)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    T, D = w.T, w.D
    out = {"cu_seqlens": w.cu_seqlens,
           "x": f32_to_bf16(rng.standard_normal((T, D), dtype=np.float32)),
           "dy": f32_to_bf16(rng.standard_normal((T, D), dtype=np.float32)),
           "w": rng.uniform(-0.5, 0.5, (D, 4)).astype(np.float32)}
    b = rng.uniform(-0.5, 0.5, D).astype(np.float32)
    halo = f32_to_bf16(rng.standard_normal((3, D), dtype=np.float32))
    if w.bias:
        out["b"] = b
    if w.halo:
        out["halo"] = halo
    return out


# ---------------------------------------------------------------- GQA attention

@dataclass(frozen=True)
class AttnWorkload:
    """Packed-varlen causal GQA attention, head dim 256: segment s has
    q_lens[s] queries and k_lens[s] keys (the causal mask is aligned to the
    bottom right of each segment)."""
    name: str
    q_lens: tuple
    k_lens: tuple
    Hq: int
    Hkv: int
    seed: int = 0
    D: int = 256

    @property
    def Tq(self) -> int:
        return int(sum(self.q_lens))

    @property
    def Tk(self) -> int:
        return int(sum(self.k_lens))

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def cu_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.k_lens)]).astype(np.int32)

    def visible_pairs(self) -> int:
        """(query, key) pairs the mask lets through, per head."""
        n = 0
        for lq, lk in zip(self.q_lens, self.k_lens):
            i = np.arange(lq)
            n += int(np.clip(i + (lk - lq) + 1, 0, lk).sum())
        return n


# The 16461-query, 24693-key layout of 8 segments with 24 query and 4 key
# heads of the pages' training-attention table; segment lengths are a fixed
# synthetic split (every segment has at least as many keys as queries).
_CP1_Q = (3150, 2604, 1987, 2411, 1503, 2216, 1330, 1260)
_CP1_EXTRA = (1024, 2048, 0, 1536, 517, 1024, 1059, 1024)

ATTN_WORKLOADS = [
    # small and ragged: a one-token segment, a segment without queries, one
    # with fewer keys than queries (its first rows see no key), one without keys
    AttnWorkload("attn_tiny", (70, 1, 0, 130, 5, 64), (100, 1, 5, 64, 0, 64), 4, 2, seed=20),
    # an odd group size (3 query heads per key head) over several blocks
    AttnWorkload("attn_grp3", (200, 65, 129), (300, 65, 200), 6, 2, seed=21),
    # plain multi-head (one query head per key head); a short query block
    # against five key blocks; a group of 4 sharing one key head
    AttnWorkload("attn_mha", (129, 3), (200, 3), 2, 2, seed=23),
    AttnWorkload("attn_longkeys", (5, 64, 1), (300, 64, 130), 4, 1, seed=24),
    # 5200 keys: the row map's sort takes three tiles and two merge passes
    AttnWorkload("attn_rowmap", (300, 200), (3000, 2200), 2, 1, seed=25),
    AttnWorkload("attn_cp1_16461", _CP1_Q, tuple(a + b for a, b in zip(_CP1_Q, _CP1_EXTRA)),
                 24, 4, seed=22),
]
ATTN_BY_NAME = {w.name: w for w in ATTN_WORKLOADS}


def make_attn_inputs(w: AttnWorkload, seed: int | None = None) -> dict:
    """q, k, v, dO as uint16 bf16 bits (standard normal), cu_q, cu_k (int32)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    return {"cu_q": w.cu_q, "cu_k": w.cu_k,
            "q": f32_to_bf16(rng.standard_normal((w.Tq, w.Hq, w.D), dtype=np.float32)),
            "k": f32_to_bf16(rng.standard_normal((w.Tk, w.Hkv, w.D), dtype=np.float32)),
            "v": f32_to_bf16(rng.standard_normal((w.Tk, w.Hkv, w.D), dtype=np.float32)),
            "dO": f32_to_bf16(rng.standard_normal((w.Tq, w.Hq, w.D), dtype=np.float32))}


def make_row_map(Tk: int, dst_rows: int, seed: int) -> np.ndarray:
    """A key-to-destination row map with repeated rows, dropped keys (-1) and
    out-of-range rows (dropped too)."""
    rng = np.random.default_rng(seed)
    m = rng.integers(0, max(dst_rows, 1), Tk).astype(np.int32)
    drop = rng.random(Tk)
    m[drop < 0.05] = -1
    m[(drop >= 0.05) & (drop < 0.07)] = dst_rows + 3
    return m
