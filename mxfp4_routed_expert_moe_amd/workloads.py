"""Seeded synthetic inputs for the MXFP4 routed-expert MoE layer.

This module only draws inputs: random bf16 activations, an fp32 router matrix,
random MXFP4 expert bytes in the canonical layout, a token-id hash table and the
token ids, and it loads the stored per-expert selection bias of the Zipf
workload.  It holds none of the layer's arithmetic (no routing, no decoding, no
GEMM), so both the CPU oracle and the HIP path can take their inputs from it.

Shapes follow the DeepSeek-V4-Flash MoE layer as the pages describe it
("DeepSeek-V4-Flash export design", Source configuration, MoE bullet): hidden
4096, 256 routed experts, top 6, intermediate 2048, one shared expert.

Canonical MXFP4 layout of one projection with N output rows and K input
columns (the reading of "ElytronAI / DeepSeek-v4-Flash", Sizes: an E2M1 nibble
plane plus one E8M0 scale per 32 columns):
  nibbles  uint8 [N, K/2]  byte b of row r holds column 2b in bits 3:0 and
                           column 2b+1 in bits 7:4
  scales   uint8 [N, K/32] E8M0 exponent of columns 32j .. 32j+31 of row r
One canonical expert is gate [I,H] | up [I,H] | down [H,I], each projection
stored as its nibble plane followed by its scale plane; experts follow each
other with no padding, the shared expert last (index E).
"""
from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np

HIDDEN = 4096
INTER = 2048
N_EXPERTS = 256
TOP_K = 6
ROUTE_SCALE = 1.5
CLAMP_LIMIT = 10.0
HASH_VOCAB = 65536

_HERE = os.path.dirname(os.path.abspath(__file__))
_REPO = os.path.dirname(_HERE)
ZIPF_BIAS_PATH = os.path.join(_REPO, "tests", "golden", "zipf_bias_e256.txt")


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    T: int
    routing: str  # "learned" or "hash"
    bias: str | None  # None or "zipf"

    @property
    def seed(self) -> int:
        return 0x5EED0000 + self.index


WORKLOADS = (
    Workload(0, "decode_t4", 4, "learned", None),
    Workload(1, "decode_t64", 64, "learned", None),
    Workload(2, "hash_t256", 256, "hash", None),
    Workload(3, "prefill_t4096", 4096, "learned", None),
    Workload(4, "prefill_t16384_zipf", 16384, "learned", "zipf"),
)


# --------------------------------------------------------------------------
# sizes of the canonical layout
# --------------------------------------------------------------------------
def projection_bytes(n_out: int, k_in: int) -> int:
    """Bytes of one canonical MXFP4 projection: nibble plane + scale plane."""
    return n_out * k_in // 2 + n_out * k_in // 32


def expert_bytes(hidden: int, inter: int) -> int:
    """Bytes of one canonical expert: gate [I,H], up [I,H], down [H,I]."""
    return 2 * projection_bytes(inter, hidden) + projection_bytes(hidden, inter)


def expert_plane_offsets(hidden: int, inter: int) -> dict:
    """Byte offsets of the six planes inside one canonical expert."""
    pg = projection_bytes(inter, hidden)
    off = {}
    off["gate_nib"] = 0
    off["gate_sc"] = inter * hidden // 2
    off["up_nib"] = pg
    off["up_sc"] = pg + inter * hidden // 2
    off["down_nib"] = 2 * pg
    off["down_sc"] = 2 * pg + hidden * inter // 2
    return off


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------
def _rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits.

    Inputs here are finite normals from a Gaussian draw, so no NaN handling.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rnd = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rnd) >> 16).astype(np.uint16)


def make_x(seed: int, T: int, hidden: int = HIDDEN) -> np.ndarray:
    """Activations: N(0,1) drawn in float32, rounded to bf16 -> uint16 [T, H]."""
    g = _rng(seed, 1)
    return f32_to_bf16_bits(g.standard_normal((T, hidden), dtype=np.float32))


def make_router(seed: int, hidden: int = HIDDEN, n_experts: int = N_EXPERTS) -> np.ndarray:
    """Router matrix W [H, E] float32 with entries N(0, 1/64)."""
    g = _rng(seed, 2)
    return (g.standard_normal((hidden, n_experts), dtype=np.float32) * np.float32(0.125)).astype(np.float32)


def make_mxfp4_expert(seed: int, xid: int, hidden: int = HIDDEN, inter: int = INTER,
                      scale_lo: int = 118, scale_hi: int = 122) -> np.ndarray:
    """Canonical bytes of MXFP4 expert xid of make_experts(seed, ...), uint8."""
    off = expert_plane_offsets(hidden, inter)
    out = np.empty(expert_bytes(hidden, inter), dtype=np.uint8)
    g = _rng(seed, 3, xid)
    for name, n, k in (("gate", inter, hidden), ("up", inter, hidden), ("down", hidden, inter)):
        o = off[name + "_nib"]
        out[o:o + n * k // 2] = np.frombuffer(g.bytes(n * k // 2), dtype=np.uint8)
        o = off[name + "_sc"]
        out[o:o + n * k // 32] = g.integers(scale_lo, scale_hi + 1, size=n * k // 32, dtype=np.uint8)
    return out


def make_experts(seed: int, n_total: int, hidden: int = HIDDEN, inter: int = INTER,
                 scale_lo: int = 118, scale_hi: int = 122) -> np.ndarray:
    """Canonical MXFP4 blob of n_total experts (routed + shared), uint8.

    Every E2M1 code is uniform over its 16 values (uniform random bytes give two
    independent uniform nibbles) and every E8M0 scale byte is uniform over
    [scale_lo, scale_hi], i.e. 2^U{-9..-5} for the default range.
    Each expert draws from its own stream, so the blob is the same whatever
    subset of it one later reads.
    """
    eb = expert_bytes(hidden, inter)
    out = np.empty(n_total * eb, dtype=np.uint8)
    for xid in range(n_total):
        out[xid * eb:(xid + 1) * eb] = make_mxfp4_expert(seed, xid, hidden, inter, scale_lo, scale_hi)
    return out


# Group sizes of the 2-bit affine codec (gate, up, down): "OsaurusAI /
# DeepSeek-V4-Flash-0731-JANG", Dynamic affine recipe.
AFFINE2_GROUPS = (64, 64, 32)


def affine2_projection_bytes(n_out: int, k_in: int, group: int) -> int:
    """Bytes of one canonical 2-bit affine projection: the code plane (four
    codes per byte) then the bf16 scale plane and the bf16 bias plane."""
    return n_out * k_in // 4 + 4 * (n_out * k_in // group)


def affine2_expert_bytes(hidden: int, inter: int) -> int:
    """Bytes of one canonical 2-bit affine expert (gate, up, down)."""
    gg, gu, gd = AFFINE2_GROUPS
    return (affine2_projection_bytes(inter, hidden, gg) + affine2_projection_bytes(inter, hidden, gu)
            + affine2_projection_bytes(hidden, inter, gd))


def make_affine2_expert(seed: int, xid: int, hidden: int = HIDDEN, inter: int = INTER) -> np.ndarray:
    """Canonical bytes of one 2-bit affine routed expert, uint8.

    Per projection [N, K] with group G: the code plane uint8 [N, K/4] (column c
    in bits 2(c%4)+1 : 2(c%4) of byte c/4; uniform random bytes make every
    code uniform over 0..3), then scales bf16 [N, K/G], then biases bf16
    [N, K/G], both little-endian.  Each group draws an exponent u uniform over
    -8..-4; its scale is 2^u (1 + f/8) with f uniform over 0..7 and its bias
    -2^u (1 + m/128) with m uniform over 0..127, so the four weight levels of a
    group straddle zero at about the MXFP4 experts' magnitude.  The bf16 bit
    patterns are drawn directly (no rounding)."""
    g = _rng(seed, 5, xid)
    out = np.empty(affine2_expert_bytes(hidden, inter), dtype=np.uint8)
    pos = 0
    for (n, k), gs in zip(((inter, hidden), (inter, hidden), (hidden, inter)), AFFINE2_GROUPS):
        out[pos:pos + n * k // 4] = np.frombuffer(g.bytes(n * k // 4), dtype=np.uint8)
        pos += n * k // 4
        ng = n * k // gs
        expo = (127 + g.integers(-8, -3, size=ng)).astype(np.uint16)
        scale = (expo << 7) | (g.integers(0, 8, size=ng).astype(np.uint16) << 4)
        bias = np.uint16(0x8000) | (expo << 7) | g.integers(0, 128, size=ng).astype(np.uint16)
        for plane in (scale, bias):
            out[pos:pos + 2 * ng] = plane.astype("<u2").view(np.uint8)
            pos += 2 * ng
    return out


def make_experts_affine2(seed: int, n_experts: int, hidden: int = HIDDEN, inter: int = INTER,
                         shared: str = "mxfp4") -> np.ndarray:
    """Canonical blob: n_experts 2-bit affine routed experts back to back, then
    the shared expert (MXFP4 expert n_experts of make_experts(seed, ...), or
    with shared="mxfp8" the make_shared_mxfp8 expert)."""
    parts = [make_affine2_expert(seed, xid, hidden, inter) for xid in range(n_experts)]
    parts.append(make_mxfp4_expert(seed, n_experts, hidden, inter) if shared == "mxfp4"
                 else make_shared_mxfp8(seed, hidden, inter))
    return np.concatenate(parts)


def mxfp8_expert_bytes(hidden: int, inter: int) -> int:
    """Bytes of one MXFP8 expert: three projections of one E4M3 byte per weight
    plus one E8M0 byte per 32 weights."""
    return 3 * hidden * inter + 3 * hidden * inter // 32


def make_shared_mxfp8(seed: int, hidden: int = HIDDEN, inter: int = INTER, scale_lo: int = 113,
                      scale_hi: int = 117) -> np.ndarray:
    """Canonical MXFP8 shared expert, uint8: per projection (gate [I,H], up [I,H],
    down [H,I]) the row-major E4M3 codes, then the [n, k/32] E8M0 scales.

    Codes are uniform over the 254 finite E4M3 codes (0x7f and 0xff, the NaN
    codes, are skipped) and scale bytes uniform over [scale_lo, scale_hi], i.e.
    2^U{-14..-10} by default, which puts the weights at about the magnitude of
    the MXFP4 experts (mean |code value| ~44 against ~2.25 for E2M1)."""
    g = _rng(seed, 4, 0)
    out = np.empty(mxfp8_expert_bytes(hidden, inter), dtype=np.uint8)
    pos = 0
    for n, k in ((inter, hidden), (inter, hidden), (hidden, inter)):
        r = g.integers(0, 254, size=n * k, dtype=np.int32)
        out[pos:pos + n * k] = (r + (r >= 0x7f) + (r >= 0xfe)).astype(np.uint8)
        pos += n * k
        out[pos:pos + n * k // 32] = g.integers(scale_lo, scale_hi + 1, size=n * k // 32, dtype=np.uint8)
        pos += n * k // 32
    return out


def make_experts_shared_mxfp8(seed: int, n_experts: int, hidden: int = HIDDEN, inter: int = INTER) -> np.ndarray:
    """Canonical blob: n_experts MXFP4 routed experts (as make_experts) followed
    by the MXFP8 shared expert (make_shared_mxfp8)."""
    return np.concatenate([make_experts(seed, n_experts, hidden, inter), make_shared_mxfp8(seed, hidden, inter)])


def make_hash(seed: int, T: int, n_experts: int = N_EXPERTS, top_k: int = TOP_K,
              vocab: int = HASH_VOCAB):
    """Token ids uniform over [0, vocab) and a table [vocab, top_k] int32 whose
    rows are top_k distinct expert ids in random order (a uniformly random
    partial permutation of 0..n_experts-1 per row)."""
    g = _rng(seed, 4)
    keys = g.random((vocab, n_experts), dtype=np.float32)
    table = np.argsort(keys, axis=1, kind="stable")[:, :top_k].astype(np.int32)
    tok = g.integers(0, vocab, size=T, dtype=np.int64).astype(np.int32)
    return np.ascontiguousarray(table), tok


def load_zipf_bias(n_experts: int = N_EXPERTS) -> np.ndarray:
    """Per-expert selection bias of the Zipf(s=1.1) workload, float32 [E].

    The stored values were written by tests/golden/make_zipf_bias.py, which
    fits them with the CPU oracle's router on a separate calibration batch.
    """
    vals = []
    with open(ZIPF_BIAS_PATH) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(float(line))
    b = np.asarray(vals, dtype=np.float32)
    if b.shape != (n_experts,):
        raise ValueError(f"{ZIPF_BIAS_PATH}: expected {n_experts} values, got {b.shape}")
    return b


@dataclass
class LayerInputs:
    workload: Workload
    x: np.ndarray            # uint16 bf16 bits [T, H]
    router: np.ndarray | None  # float32 [H, E]
    bias: np.ndarray | None    # float32 [E]
    table: np.ndarray | None   # int32 [V, k]
    tok: np.ndarray | None     # int32 [T]
    experts: np.ndarray        # uint8 canonical blob, (E + 1) experts
    hidden: int
    inter: int
    n_experts: int
    top_k: int


def make_layer_inputs(w: Workload, T: int | None = None, hidden: int = HIDDEN, inter: int = INTER,
                      n_experts: int = N_EXPERTS, top_k: int = TOP_K, experts: np.ndarray | None = None) -> LayerInputs:
    """All inputs of one workload (T may be overridden for a reduced sample)."""
    T = w.T if T is None else T
    x = make_x(w.seed, T, hidden)
    router = bias = table = tok = None
    if w.routing == "learned":
        router = make_router(w.seed, hidden, n_experts)
        if w.bias == "zipf":
            bias = load_zipf_bias(n_experts)
    else:
        table, tok = make_hash(w.seed, T, n_experts, top_k)
    if experts is None:
        experts = make_experts(w.seed, n_experts + 1, hidden, inter)
    return LayerInputs(w, x, router, bias, table, tok, experts, hidden, inter, n_experts, top_k)
