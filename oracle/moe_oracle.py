"""CPU oracle of the MXFP4 routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import or call this module.  The product path (the HIP library and its Python
binding) never does, and this module shares no code with it: it has its own
E2M1 table, its own reader of the canonical byte layout and its own loops.

Plain and slow on purpose: numpy in float64, one expert at a time, no blocking
or fusion.  A library matmul (numpy's float64 GEMM) serves as the dot-product
step; every product of a bf16 activation and a decoded MXFP4 weight is exact in
float64, so only the summation order differs from any other correct
implementation.

What the layer computes, with the passage each step follows:

* Router ("Model techniques map -- DeepSeek-V4-Flash", Checked in its code,
  rows "Mixture of experts" and "Auxiliary-loss-free load balancing";
  "DeepSeek-V4-Flash export design", Source configuration, MoE bullet):
  logits z = x W with the router kept in float32 storage, score
  s = sqrt(softplus(z)), selection of the top 6 of s + b where the bias b only
  changes which experts are chosen, weights gathered from the unbiased s,
  normalised over the chosen six and scaled by 1.5.
* Hash routing (same MoE bullet; "EasyDeL / DeepSeek-V4-Flash", Architecture):
  the expert ids of a token are a row of a token-id table.
* Experts (techniques map, row "SwiGLU feed-forward"): down(silu(min(gate(x), L))
  * clamp(up(x), -L, L)); weights are MXFP4 ("ElytronAI / DeepSeek-v4-Flash",
  Sizes: E2M1 codes with one E8M0 scale per group of 32 columns).
* Shared expert and combine (techniques map, row "Shared expert"): the routed
  outputs weighted and summed, plus the shared expert applied to the same input.
* Optionally the routed experts in the 2-bit affine codec ("OsaurusAI /
  DeepSeek-V4-Flash-0731-JANG", Dynamic affine recipe): weight = s * q + b
  with a 2-bit code q and one (s, b) per group of consecutive input columns,
  64 for gate and up, 32 for down.
* Optionally the shared expert in MXFP8 ("ElytronAI / DeepSeek-v4-Flash",
  Sizes: the dense weights as E4M3 with one E8M0 scale per 32 columns, the
  mxfp8_lt re-encode), otherwise in MXFP4 like the routed experts.

Readings where the pages are silent (each also listed with the design notes):
E2M1/E8M0 bit meaning per the OCP microscaling formats; low nibble = even
column; scale groups run along the input (reduction) axis; ties in the top-6
go to the lower expert id and the six come out in descending key order;
softplus is the exact stable form; hash weights are 1.5/6; the shared expert
has weight 1 and is stored as expert E; h = silu(.)*clamp(.) is rounded to
bf16 before the down projection; dispatch order is (expert, token, slot);
affine codes are unsigned, four to a byte with column c in bits 2(c%4)+1:2(c%4)
of byte c/4, and s, b are bf16 (the codec's scales, biases: MLX affine form).

Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, brute force, invariants).  Full-layer outputs have no worked
numeric example on the pages; they are pinned through those checks only.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
# E2M1 code -> value: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0.
# Codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 are their negatives.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def _e4m3_table() -> np.ndarray:
    """E4M3 code -> value (OCP FP8 E4M3, the variant without infinities):
    sign bit 7, exponent bits 6:3 with bias 7, mantissa bits 2:0.  Exponent 0
    is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN, so the
    largest finite magnitude is 1.75 * 2^8 = 448."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e8m0_value(e) -> np.ndarray:
    """E8M0 scale byte -> 2^(e-127) in float64 (exact); 255 is NaN."""
    e = np.asarray(e, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), returned
    as float64.  Single rounding straight from float64, subnormals kept
    (bf16 has 8 significant bits and the float32 exponent range)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    fin = np.isfinite(v)
    a = np.abs(v[fin])
    _, ex = np.frexp(a)             # a = m * 2^ex, m in [0.5, 1)
    ex = np.maximum(ex, -125)       # below 2^-126 the quantum stays 2^-133
    q = np.ldexp(1.0, ex - 8)       # spacing of 8-bit significands in [2^(ex-1), 2^ex)
    r = np.rint(a / q) * q          # np.rint rounds half to even; a/q is exact
    r = np.where(r >= 2.0 ** 128 - 2.0 ** 119, np.inf, r)  # beyond max bf16 rounds to inf
    out[fin] = np.copysign(r, v[fin])
    out[~fin] = v[~fin]
    return out


# --------------------------------------------------------------------------
# canonical MXFP4 reader
# --------------------------------------------------------------------------
def decode_mxfp4(nibbles: np.ndarray, scales: np.ndarray, n_out: int, k_in: int) -> np.ndarray:
    """Decode one canonical projection to float64 [n_out, k_in].

    W[r, c] = E2M1(code of column c in row r) * 2^(scale[r, c // 32] - 127).
    """
    nib = np.asarray(nibbles, dtype=np.uint8).reshape(n_out, k_in // 2)
    sc = np.asarray(scales, dtype=np.uint8).reshape(n_out, k_in // 32)
    codes = np.empty((n_out, k_in), dtype=np.uint8)
    codes[:, 0::2] = nib & 0x0F
    codes[:, 1::2] = nib >> 4
    w = E2M1_VALUES[codes].reshape(n_out, k_in // 32, 32)
    w *= e8m0_value(sc)[:, :, None]
    return w.reshape(n_out, k_in)


def decode_mxfp8(codes: np.ndarray, scales: np.ndarray, n_out: int, k_in: int) -> np.ndarray:
    """Decode one canonical MXFP8 projection to float64 [n_out, k_in]:
    W[r, c] = E4M3(code[r, c]) * 2^(scale[r, c // 32] - 127), one code byte
    per weight in row-major order, then the [n_out, k_in / 32] scale bytes."""
    cd = np.asarray(codes, dtype=np.uint8).reshape(n_out, k_in)
    sc = np.asarray(scales, dtype=np.uint8).reshape(n_out, k_in // 32)
    w = E4M3_VALUES[cd].reshape(n_out, k_in // 32, 32)
    w *= e8m0_value(sc)[:, :, None]
    return w.reshape(n_out, k_in)


# Group sizes of the 2-bit affine codec, per projection (gate, up, down):
# "OsaurusAI / DeepSeek-V4-Flash-0731-JANG", Dynamic affine recipe.
AFFINE2_GROUPS = (64, 64, 32)


def decode_affine2(codes: np.ndarray, scales: np.ndarray, biases: np.ndarray, n_out: int, k_in: int,
                   group: int) -> np.ndarray:
    """Decode one canonical 2-bit affine projection to float64 [n_out, k_in]:
    W[r, c] = s[r, c // G] * q[r, c] + b[r, c // G], q the 2-bit code of column c
    (bits 2(c%4)+1 : 2(c%4) of byte c // 4 of row r), s and b bf16 [n_out, k_in / G].
    Exact in float64 (q <= 3, s and b have 8 significant bits)."""
    cb = np.asarray(codes, dtype=np.uint8).reshape(n_out, k_in // 4)
    q = np.empty((n_out, k_in), dtype=np.float64)
    for j in range(4):
        q[:, j::4] = (cb >> (2 * j)) & 3
    s = bf16_bits_to_f64(np.asarray(scales, dtype=np.uint8).view("<u2").reshape(n_out, k_in // group))
    b = bf16_bits_to_f64(np.asarray(biases, dtype=np.uint8).view("<u2").reshape(n_out, k_in // group))
    return (q.reshape(n_out, k_in // group, group) * s[:, :, None] + b[:, :, None]).reshape(n_out, k_in)


def canonical_affine2_expert_size(hidden: int, inter: int) -> int:
    """Bytes of one canonical 2-bit affine expert: per projection its code plane
    (2 bits per weight) then its bf16 scale plane and bf16 bias plane."""
    proj = lambda n, k, gs: n * k // 4 + 4 * (n * k // gs)  # noqa: E731
    gg, gu, gd = AFFINE2_GROUPS
    return proj(inter, hidden, gg) + proj(inter, hidden, gu) + proj(hidden, inter, gd)


def canonical_expert_size(hidden: int, inter: int) -> int:
    """Bytes of one canonical expert (gate, up, down; 4.25 bits per weight)."""
    proj = lambda n, k: n * k // 2 + n * k // 32  # noqa: E731
    return 2 * proj(inter, hidden) + proj(hidden, inter)


def canonical_mxfp8_expert_size(hidden: int, inter: int) -> int:
    """Bytes of one canonical MXFP8 expert (gate, up, down; 8.25 bits per weight)."""
    proj = lambda n, k: n * k + n * k // 32  # noqa: E731
    return 2 * proj(inter, hidden) + proj(hidden, inter)


def decode_expert(blob: np.ndarray, xid: int, hidden: int, inter: int, fmt: str = "mxfp4",
                  routed_fmt: str = "mxfp4"):
    """Decode expert xid of a canonical blob -> (gate [I,H], up [I,H], down [H,I]).

    The routed experts sit back to back in routed_fmt ("mxfp4" or "affine2"),
    so expert xid starts at xid times the size of one routed expert; fmt is the
    format of expert xid itself ("mxfp8" reads an MXFP8 expert there: the
    shared expert stored last, after the routed ones)."""
    eb = canonical_affine2_expert_size(hidden, inter) if routed_fmt == "affine2" else canonical_expert_size(hidden, inter)
    pos = xid * eb
    mats = []
    for (n, k), gs in zip(((inter, hidden), (inter, hidden), (hidden, inter)), AFFINE2_GROUPS):
        if fmt == "affine2":
            nc, ns = n * k // 4, 2 * (n * k // gs)
            mats.append(decode_affine2(blob[pos:pos + nc], blob[pos + nc:pos + nc + ns],
                                       blob[pos + nc + ns:pos + nc + 2 * ns], n, k, gs))
            pos += nc + 2 * ns
            continue
        if fmt == "mxfp4":
            nn, ns = n * k // 2, n * k // 32
            mats.append(decode_mxfp4(blob[pos:pos + nn], blob[pos + nn:pos + nn + ns], n, k))
        elif fmt == "mxfp8":
            nn, ns = n * k, n * k // 32
            mats.append(decode_mxfp8(blob[pos:pos + nn], blob[pos + nn:pos + nn + ns], n, k))
        else:
            raise ValueError(f"unknown weight format {fmt!r}")
        pos += nn + ns
    return tuple(mats)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def sqrt_softplus(z: np.ndarray) -> np.ndarray:
    """s = sqrt(log(1 + e^z)) with the overflow-free form max(z,0) + log1p(e^-|z|)."""
    z = np.asarray(z, dtype=np.float64)
    return np.sqrt(np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z))))


def router_logits(x_bits: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """z[t, e] = sum_h x[t, h] * W[h, e], float64 products and sums."""
    return bf16_bits_to_f64(x_bits) @ np.asarray(w_router, dtype=np.float32).astype(np.float64)


def select_top_k(key: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row, descending; equal keys -> lower index
    first (a stable sort of -key keeps the lower index ahead)."""
    order = np.argsort(-key, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def route_learned(x_bits, w_router, bias, top_k: int, route_scale: float):
    """Learned routing -> (ids int32 [T,k], weights float64 [T,k], scores float64 [T,E])."""
    z = router_logits(x_bits, w_router)
    s = sqrt_softplus(z)
    key = s if bias is None else s + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    ids = select_top_k(key, top_k)
    sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    w = route_scale * sel / sel.sum(axis=1, keepdims=True)
    return ids, w, s


def route_hash(token_ids, table, top_k: int, route_scale: float):
    """Hash routing: ids = table[token]; every weight route_scale / top_k."""
    tok = np.asarray(token_ids, dtype=np.int64)
    ids = np.asarray(table, dtype=np.int32)[tok, :top_k].copy()
    w = np.full(ids.shape, route_scale / top_k, dtype=np.float64)
    return ids, w


def boundary_gap(x_bits, w_router, bias, top_k: int) -> np.ndarray:
    """Per token, key[k-th] - key[(k+1)-th] (float64).  A tiny gap means the
    selection sits on a near tie and either set is a correct answer.  With
    top_k equal to the expert count every expert is chosen: no boundary, gap +inf."""
    s = sqrt_softplus(router_logits(x_bits, w_router))
    key = s if bias is None else s + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    if top_k >= key.shape[1]:
        return np.full(key.shape[0], np.inf)
    part = -np.sort(-key, axis=1)
    return part[:, top_k - 1] - part[:, top_k]


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------
def dispatch(ids: np.ndarray, n_experts: int):
    """Group the (token, slot) pairs by expert, stably in (expert, token, slot)
    order, and append the shared-expert group (every token, in order).

    Returns offsets int32 [E+2] (group g holds rows offsets[g]..offsets[g+1]-1,
    group E is the shared expert), row_token int32 [rows] and slot_row int32
    [T, k+1] (row of pair (t, j); column k is the shared row).  Ids outside
    [0, E) are dropped: they get no row and slot_row -1.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < n_experts)
    pair = np.nonzero(valid)[0]                       # (t, j) flat indices, ascending
    order = pair[np.argsort(flat[pair], kind="stable")]
    counts = np.bincount(flat[pair], minlength=n_experts)
    offsets = np.zeros(n_experts + 2, dtype=np.int64)
    offsets[1:n_experts + 1] = np.cumsum(counts)
    n_routed = int(offsets[n_experts])
    offsets[n_experts + 1] = n_routed + T
    row_token = np.empty(n_routed + T, dtype=np.int64)
    row_token[:n_routed] = order // k
    row_token[n_routed:] = np.arange(T)
    routed_row = np.full(T * k, -1, dtype=np.int64)
    routed_row[order] = np.arange(n_routed)
    slot_row = np.empty((T, k + 1), dtype=np.int64)
    slot_row[:, :k] = routed_row.reshape(T, k)
    slot_row[:, k] = n_routed + np.arange(T)
    return offsets.astype(np.int32), row_token.astype(np.int32), slot_row.astype(np.int32)


# --------------------------------------------------------------------------
# experts and combine
# --------------------------------------------------------------------------
def silu(v: np.ndarray) -> np.ndarray:
    """silu(v) = v / (1 + e^-v) in float64."""
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def swiglu_clamped(g: np.ndarray, u: np.ndarray, limit: float) -> np.ndarray:
    """silu(min(g, L)) * min(max(u, -L), L): gate clamped above only, up on both sides."""
    return silu(np.minimum(g, limit)) * np.clip(u, -limit, limit)


def expert_forward(xf: np.ndarray, mats, limit: float) -> np.ndarray:
    """One expert on float64 rows xf [m, H] -> float64 [m, H]; h rounded to bf16."""
    wg, wu, wd = mats
    g = xf @ wg.T
    u = xf @ wu.T
    h = round_to_bf16(swiglu_clamped(g, u, limit))
    return h @ wd.T


def expert_ffn(x_bits, blob, offsets, row_token, limit: float, n_experts: int, hidden: int, inter: int,
               groups=None, shared_fmt: str = "mxfp4", routed_fmt: str = "mxfp4") -> np.ndarray:
    """Every dispatched row through its expert -> float64 [rows, H].

    Expert-major: each group with rows is decoded once, then its rows run.
    `groups` optionally restricts the work to some groups (other rows stay 0);
    shared_fmt is the weight format of the shared expert (group n_experts),
    routed_fmt that of the routed ones.
    """
    xf = bf16_bits_to_f64(x_bits)
    offsets = np.asarray(offsets, dtype=np.int64)
    row_token = np.asarray(row_token, dtype=np.int64)
    out = np.zeros((int(offsets[-1]), hidden), dtype=np.float64)
    for g in (range(n_experts + 1) if groups is None else groups):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 == r0:
            continue
        mats = decode_expert(blob, g, hidden, inter, shared_fmt if g == n_experts else routed_fmt, routed_fmt)
        out[r0:r1] = expert_forward(xf[row_token[r0:r1]], mats, limit)
    return out


def combine(out_rows: np.ndarray, slot_row: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """y[t] = sum_j w[t, j] * out[slot_row[t, j]] (j < k, in slot order) + out[shared row of t].

    Slots whose row is -1 (dropped ids) contribute nothing.  float64."""
    slot_row = np.asarray(slot_row, dtype=np.int64)
    T, kp1 = slot_row.shape
    k = kp1 - 1
    H = out_rows.shape[1]
    y = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        r = slot_row[:, j]
        ok = r >= 0
        y[ok] += np.asarray(weights, dtype=np.float64)[ok, j:j + 1] * out_rows[r[ok]]
    y += out_rows[slot_row[:, k]]
    return y


def moe_layer(x_bits, blob, *, n_experts: int, hidden: int, inter: int, top_k: int,
              route_scale: float, limit: float, w_router=None, bias=None, token_ids=None, table=None,
              shared_fmt: str = "mxfp4", routed_fmt: str = "mxfp4"):
    """The whole layer: route -> dispatch -> expert FFN -> combine.  Returns a dict
    with ids, weights, offsets, row_token, slot_row, out_rows and y (float64)."""
    if table is not None:
        ids, w = route_hash(token_ids, table, top_k, route_scale)
    else:
        ids, w, _ = route_learned(x_bits, w_router, bias, top_k, route_scale)
    offsets, row_token, slot_row = dispatch(ids, n_experts)
    out = expert_ffn(x_bits, blob, offsets, row_token, limit, n_experts, hidden, inter, shared_fmt=shared_fmt,
                     routed_fmt=routed_fmt)
    y = combine(out, slot_row, w)
    return dict(ids=ids, weights=w, offsets=offsets, row_token=row_token, slot_row=slot_row,
                out_rows=out, y=y)


def dense_moe_layer(x_bits, blob, ids, weights, *, n_experts: int, hidden: int, inter: int, limit: float,
                    shared_fmt: str = "mxfp4", routed_fmt: str = "mxfp4"):
    """Brute force without dispatch: every token through ALL experts, masked by a
    0/1 selection mask and weighted, plus the shared expert.  Tiny inputs only."""
    xf = bf16_bits_to_f64(x_bits)
    T = xf.shape[0]
    ids = np.asarray(ids, dtype=np.int64)
    y = np.zeros((T, hidden), dtype=np.float64)
    for e in range(n_experts):
        mask = (ids == e)                               # [T, k]
        we = (np.asarray(weights, dtype=np.float64) * mask).sum(axis=1)  # 0 where not chosen
        sel = mask.any(axis=1).astype(np.float64)
        ye = expert_forward(xf, decode_expert(blob, e, hidden, inter, routed_fmt, routed_fmt), limit)
        y += (sel * we)[:, None] * ye
    y += expert_forward(xf, decode_expert(blob, n_experts, hidden, inter, shared_fmt, routed_fmt), limit)
    return y
