"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each check reaches the value
another way (the format's bit-field definition, high-precision decimal
arithmetic, brute force in plain Python, exact invariants, closed-form experts,
torch's own bf16 conversion) so that a dropped term, a wrong sign or index or a
transposed operand in the oracle fails one of them.
"""
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from mxfp4_routed_expert_moe_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_constants():
    vals = {}
    with open(os.path.join(GOLDEN, "page_constants.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (s.strip() for s in line.split("="))
                vals[k] = float(v) if "." in v else int(v)
    return vals


# ---------------------------------------------------------------- formats
def test_e2m1_table_from_bit_fields():
    # E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa; exponent 0 is subnormal.
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
        want = -mag if s else mag
        got = O.E2M1_VALUES[code]
        assert got == want and math.copysign(1.0, got) == (-1.0 if s else 1.0), code
    assert O.E2M1_VALUES.max() == 6.0 and O.E2M1_VALUES[1] == 0.5


@pytest.mark.parametrize("e", [0, 1, 118, 119, 120, 121, 122, 127, 200, 252, 254])
def test_e8m0_scale_and_decode_exact(e):
    v = O.e8m0_value(e)
    assert v == math.ldexp(1.0, e - 127)
    # every code times every scale decodes exactly; also into float32 where it fits
    nib = np.array([[0x10 | 0x0, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] * 2], dtype=np.uint8)
    w = O.decode_mxfp4(nib, np.array([[e]], dtype=np.uint8), 1, 32)[0]
    codes = [c for b in nib[0] for c in (b & 15, b >> 4)]
    for c, got in zip(codes, w):
        s, ee, m = c >> 3, (c >> 1) & 3, c & 1
        mag = (m * 0.5) if ee == 0 else (2.0 ** (ee - 1)) * (1.0 + m / 2.0)
        want = math.ldexp(-mag if s else mag, e - 127)
        assert got == want
        if e <= 252:
            assert float(np.float32(got)) == got  # exact in float32 (0.5*2^-127 is a subnormal)


def test_e8m0_255_is_nan():
    assert np.isnan(O.e8m0_value(255))


def test_nibble_order_and_scale_axis():
    # row 0: byte 0 = 0x21 -> column 0 code 1 (0.5), column 1 code 2 (1.0)
    # groups of 32 columns take their own scale: scale bytes 127, 128 -> x1, x2
    nib = np.zeros((2, 32), dtype=np.uint8)
    nib[0, 0] = 0x21
    nib[0, 16] = 0x43      # column 32 -> code 3 (1.5), column 33 -> code 4 (2.0)
    nib[1, 31] = 0xF0      # row 1: column 62 -> 0, column 63 -> code 15 (-6)
    sc = np.array([[127, 128], [126, 129]], dtype=np.uint8)
    w = O.decode_mxfp4(nib, sc, 2, 64)
    assert w[0, 0] == 0.5 and w[0, 1] == 1.0
    assert w[0, 32] == 1.5 * 2 and w[0, 33] == 2.0 * 2
    assert w[1, 62] == 0.0 and w[1, 63] == -6.0 * 4
    assert np.count_nonzero(w) == 5


def test_page_byte_arithmetic():
    c = _page_constants()
    H, I, E = c["hidden"], c["intermediate"], c["n_routed_experts"]
    g = c["scale_group"]
    per_proj = H * I // 2 + H * I // g
    assert per_proj == 4_456_448
    assert O.canonical_expert_size(H, I) == 3 * per_proj == 13_369_344
    layers = c["routed_expert_projections"] // 3
    assert layers * 3 == c["routed_expert_projections"]
    assert O.canonical_expert_size(H, I) * E * layers == c["expert_payload_bytes"]
    # 4.25 bits per weight, no padding
    assert O.canonical_expert_size(H, I) * 8 == 3 * H * I * 4.25
    # the generator's layout agrees with the oracle's reader
    assert WL.expert_bytes(H, I) == O.canonical_expert_size(H, I)


def test_page_hyperparameters_match_workloads():
    c = _page_constants()
    assert (WL.HIDDEN, WL.N_EXPERTS, WL.TOP_K, WL.INTER, WL.ROUTE_SCALE) == (
        c["hidden"], c["n_routed_experts"], c["top_k"], c["intermediate"], c["route_scale"])
    assert c["n_shared_experts"] == 1


# ---------------------------------------------------------------- bf16
def test_bf16_bits_to_f64_matches_torch():
    g = np.random.default_rng(1)
    bits = g.integers(0, 1 << 16, 20000, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    o = O.bf16_bits_to_f64(bits)
    same = (o == t) | (np.isnan(o) & np.isnan(t))
    assert same.all()


def test_round_to_bf16_matches_torch_on_float32_values():
    # For values that are float32 numbers, rounding straight from float64 is the
    # same as torch's float32 -> bf16 round-to-nearest-even.
    g = np.random.default_rng(2)
    f = np.concatenate([
        g.standard_normal(50000).astype(np.float32) * np.float32(7.0),
        (g.standard_normal(5000) * 1e-39).astype(np.float32),          # subnormals
        g.integers(0, 1 << 32, 50000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_to_bf16_ties_and_overflow():
    assert O.round_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0               # tie -> even
    assert O.round_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6  # tie -> even
    assert O.round_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1 + 2.0 ** -7
    assert O.round_to_bf16(np.array([-(1 + 2.0 ** -8 + 2.0 ** -40)]))[0] == -(1 + 2.0 ** -7)
    big = (2 - 2.0 ** -7) * 2.0 ** 127
    assert O.round_to_bf16(np.array([big]))[0] == big
    assert O.round_to_bf16(np.array([2.0 ** 128 - 2.0 ** 119]))[0] == np.inf
    assert O.round_to_bf16(np.array([2.0 ** -133 * 0.75]))[0] == 2.0 ** -133


# ---------------------------------------------------------------- scalar functions
def _dec_softplus_sqrt(z):
    getcontext().prec = 60
    d = Decimal(z)
    return float((Decimal(1) + d.exp()).ln().sqrt())


def _dec_silu(v):
    getcontext().prec = 60
    d = Decimal(v)
    return float(d / (Decimal(1) + (-d).exp()))


def test_sqrt_softplus_against_decimal():
    zs = [0.0, 1e-8, -1e-8, 0.5, -0.5, 1.0, -3.0, 7.25, -7.25, 20.0, -20.0, 35.5, -35.5, 80.0, -80.0, 700.0]
    got = O.sqrt_softplus(np.array(zs))
    for z, g in zip(zs, got):
        assert g == pytest.approx(_dec_softplus_sqrt(z), rel=4e-16), z
    assert got[0] == pytest.approx(math.sqrt(math.log(2.0)), rel=1e-16)


def test_silu_and_clamp_against_decimal():
    vs = [0.0, 1.0, -1.0, 3.5, -3.5, 9.99, 10.0, 12.0, -12.0, 40.0, -40.0, -800.0]
    got = O.silu(np.array(vs))
    for v, g in zip(vs, got):
        assert g == pytest.approx(_dec_silu(v), rel=4e-16, abs=1e-300), v
    L = 10.0
    g = np.array([12.0, -12.0, 9.99, 3.0])
    u = np.array([-12.0, 12.0, 9.99, -3.0])
    h = O.swiglu_clamped(g, u, L)
    # gate clamped above only, up clamped both sides
    want = [_dec_silu(10.0) * -10.0, _dec_silu(-12.0) * 10.0, _dec_silu(9.99) * 9.99, _dec_silu(3.0) * -3.0]
    assert np.allclose(h, want, rtol=1e-15, atol=0)


# ---------------------------------------------------------------- routing
def _small_routing_inputs(T=40, H=128, E=32, seed=11):
    g = np.random.default_rng(seed)
    x = WL.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    w = (g.standard_normal((H, E)) * 0.125).astype(np.float32)
    return x, w


def test_router_logits_against_exact_sum():
    x, w = _small_routing_inputs()
    z = O.router_logits(x, w)
    xf = O.bf16_bits_to_f64(x)
    for t, e in [(0, 0), (3, 17), (39, 31), (20, 5)]:
        terms = [float(xf[t, h]) * float(w[h, e]) for h in range(x.shape[1])]  # exact products
        exact = math.fsum(terms)
        assert abs(z[t, e] - exact) <= 64 * 2.0 ** -53 * math.fsum(abs(v) for v in terms)


@pytest.mark.parametrize("bias_kind", ["none", "random"])
def test_learned_routing_brute_force(bias_kind):
    x, w = _small_routing_inputs()
    E, k = w.shape[1], 6
    bias = None if bias_kind == "none" else np.random.default_rng(5).standard_normal(E).astype(np.float32)
    ids, wt, s = O.route_learned(x, w, bias, k, 1.5)
    xf = O.bf16_bits_to_f64(x)
    for t in range(x.shape[0]):
        keys = []
        for e in range(E):
            z = math.fsum(float(xf[t, h]) * float(w[h, e]) for h in range(x.shape[1]))
            sc = _dec_softplus_sqrt(z)
            keys.append((-(sc + (0.0 if bias is None else float(bias[e]))), e, sc))
        keys.sort()
        want = [e for _, e, _ in keys[:k]]
        assert list(ids[t]) == want
        ssel = [sc for _, _, sc in keys[:k]]
        for j in range(k):
            assert wt[t, j] == pytest.approx(1.5 * ssel[j] / math.fsum(ssel), rel=1e-13)
        assert abs(wt[t].sum() - 1.5) <= 1e-12


def test_boundary_gap_hand_built_keys():
    # A zero router gives every expert the same score sqrt(log 2); the
    # selection keys are then that score plus a bias of exact binary
    # fractions, so the gap between the k-th and (k+1)-th largest key is a
    # difference of two biases, known in closed form (each key is one float64
    # rounding of score + bias away from exact: 2^-52 at most).
    E, H = 16, 512
    x = WL.make_x(11, 3, H)
    w = np.zeros((H, E), dtype=np.float32)
    b = np.zeros(E, dtype=np.float32)
    b[[4, 9, 1, 12, 2, 14, 7, 3]] = [1.0, 0.75, 0.5, 0.375, 0.25, 0.125, 0.0625, 0.03125]
    # sorted biases: 1, .75, .5, .375, .25, .125 | .0625, .03125, 0 (x8)
    for k, want in ((6, 0.125 - 0.0625), (3, 0.5 - 0.375), (1, 1.0 - 0.75), (8, 0.03125), (9, 0.0)):
        gap = O.boundary_gap(x, w, b, k)
        assert gap.shape == (3,)
        assert np.all(np.abs(gap - want) <= 2.0 ** -50), (k, gap, want)
    # an exact tie across the boundary: the 6th and 7th keys are equal
    b2 = b.copy()
    b2[7] = 0.125
    assert np.all(O.boundary_gap(x, w, b2, 6) == 0.0)
    # the gap is on the biased keys: without the bias every key is equal
    assert np.all(O.boundary_gap(x, w, None, 6) == 0.0)


@pytest.mark.parametrize("bias_kind", ["none", "random"])
def test_boundary_gap_brute_force(bias_kind):
    # keys from exactly summed logits and a 60-digit decimal sqrt-softplus,
    # sorted in plain Python; the gap between the k-th and (k+1)-th largest
    x, w = _small_routing_inputs()
    E = w.shape[1]
    bias = None if bias_kind == "none" else np.random.default_rng(9).standard_normal(E).astype(np.float32)
    xf = O.bf16_bits_to_f64(x)
    for k in (1, 6):
        gap = O.boundary_gap(x, w, bias, k)
        for t in range(0, x.shape[0], 3):
            keys = []
            for e in range(E):
                z = math.fsum(float(xf[t, h]) * float(w[h, e]) for h in range(x.shape[1]))
                keys.append(_dec_softplus_sqrt(z) + (0.0 if bias is None else float(bias[e])))
            keys.sort(reverse=True)
            want = keys[k - 1] - keys[k]
            assert want > 0
            assert abs(gap[t] - want) <= 1e-12 * max(1.0, abs(keys[0])), (k, t, gap[t], want)


def test_selection_bias_only_selects():
    # +1e6 on six chosen experts forces exactly those; their weights still come
    # from the unbiased scores (selection bias changes choice, not weights).
    x, w = _small_routing_inputs()
    E = w.shape[1]
    chosen = [3, 29, 7, 0, 18, 11]
    bias = np.zeros(E, dtype=np.float32)
    bias[chosen] = 1e6
    ids, wt, s = O.route_learned(x, w, bias, 6, 1.5)
    ids0, wt0, s0 = O.route_learned(x, w, None, 6, 1.5)
    for t in range(x.shape[0]):
        assert sorted(ids[t]) == sorted(chosen)
        sel = s0[t, ids[t]]
        assert np.allclose(wt[t], 1.5 * sel / sel.sum(), rtol=1e-15)
        # descending unbiased score among the forced set (equal bias)
        assert all(sel[j] >= sel[j + 1] for j in range(5))


def test_top_k_ties_go_to_lower_id():
    key = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 0.5, 2.0, 2.0]])
    assert list(O.select_top_k(key, 6)[0]) == [1, 2, 4, 3, 6, 7]


def test_hash_routing_is_table_lookup():
    table, tok = WL.make_hash(123, 300)
    ids, w = O.route_hash(tok, table, 6, 1.5)
    for t in range(300):
        assert list(ids[t]) == list(table[tok[t]])
        assert len(set(ids[t])) == 6
    assert np.all(w == 1.5 / 6)


# ---------------------------------------------------------------- dispatch
def _dispatch_brute(ids, E):
    T, k = len(ids), len(ids[0])
    rows = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t][j] == e:
                    rows.append((e, t, j))
    return rows


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dispatch_brute_force(seed):
    g = np.random.default_rng(seed)
    T, k, E = 37, 6, 16
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if seed == 2:
        ids[5, 3] = ids[5, 1]          # a repeated id inside one token still dispatches stably
        ids[9, 0] = E + 3              # out-of-range ids are dropped
        ids[10, 4] = -1
    offsets, row_token, slot_row = O.dispatch(ids, E)
    rows = _dispatch_brute(ids.tolist(), E)
    n_routed = len(rows)
    assert offsets[0] == 0 and offsets[E] == n_routed and offsets[E + 1] == n_routed + T
    for e in range(E):
        assert offsets[e + 1] - offsets[e] == sum(1 for r in rows if r[0] == e)
    for p, (e, t, j) in enumerate(rows):
        assert row_token[p] == t and slot_row[t, j] == p and offsets[e] <= p < offsets[e + 1]
    assert list(row_token[n_routed:]) == list(range(T))
    assert list(slot_row[:, k]) == list(range(n_routed, n_routed + T))
    valid = (ids >= 0) & (ids < E)
    assert np.all(slot_row[:, :k][~valid] == -1)
    assert sorted(slot_row[:, :k][valid].tolist()) == list(range(n_routed))


# ---------------------------------------------------------------- experts
def _identity_experts(hidden, inter, n_total, up_code=0x2, down_exp=127):
    """gate = [I_inter | 0] (code 2 = 1.0 on the diagonal), up = up_code on the
    diagonal, down = [I_inter ; 0]; all scales 2^0 except down's (down_exp)."""
    eb = O.canonical_expert_size(hidden, inter)
    blob = np.zeros(n_total * eb, dtype=np.uint8)
    off = WL.expert_plane_offsets(hidden, inter)
    for xid in range(n_total):
        b = xid * eb
        for name, code in (("gate", 0x2), ("up", up_code)):
            nib = blob[b + off[name + "_nib"]: b + off[name + "_nib"] + inter * hidden // 2].reshape(inter, hidden // 2)
            for i in range(inter):
                nib[i, i // 2] |= code << (4 * (i & 1))
            blob[b + off[name + "_sc"]: b + off[name + "_sc"] + inter * hidden // 32] = 127
        nib = blob[b + off["down_nib"]: b + off["down_nib"] + hidden * inter // 2].reshape(hidden, inter // 2)
        for i in range(inter):
            nib[i, i // 2] |= 0x2 << (4 * (i & 1))
        blob[b + off["down_sc"]: b + off["down_sc"] + hidden * inter // 32] = down_exp
    return blob


def _clamp_inputs(T, hidden):
    g = np.random.default_rng(3)
    xf = g.standard_normal((T, hidden)).astype(np.float32) * 4
    xf[0, :6] = [12.0, -12.0, 9.99, -9.99, 10.0, -10.0]   # both clamp branches fire
    return WL.f32_to_bf16_bits(xf)


@pytest.mark.parametrize("shape", [(64, 32), (4096, 2048)])
def test_identity_expert_closed_form(shape):
    hidden, inter = shape
    L = 10.0
    blob = _identity_experts(hidden, inter, 1)
    x = _clamp_inputs(3, hidden)
    xf = O.bf16_bits_to_f64(x)
    o = O.expert_forward(xf, O.decode_expert(blob, 0, hidden, inter), L)
    v = xf[:, :inter]
    want = np.array([[_dec_silu(min(a, L)) * max(min(a, L), -L) for a in row] for row in v])
    # h is rounded to bf16: within half a bf16 ulp (2^-8 relative)
    assert np.all(np.abs(o[:, :inter] - want) <= 2.0 ** -8 * np.abs(want) + 1e-300)
    assert np.all(o[:, inter:] == 0.0)
    assert o[0, 0] == O.round_to_bf16(np.array([_dec_silu(10.0) * 10.0]))[0]


def test_gate_up_orientation():
    # gate = I, up = 2I must give silu(min(x,L)) * clamp(2x,-L,L), not the swap
    hidden, inter, L = 64, 32, 10.0
    blob = _identity_experts(hidden, inter, 1, up_code=0x4)
    x = _clamp_inputs(4, hidden)
    xf = O.bf16_bits_to_f64(x)
    o = O.expert_forward(xf, O.decode_expert(blob, 0, hidden, inter), L)[:, :inter]
    v = xf[:, :inter]
    right = np.vectorize(lambda a: _dec_silu(min(a, L)) * max(min(2 * a, L), -L))(v)
    swapped = np.vectorize(lambda a: _dec_silu(min(2 * a, L)) * max(min(a, L), -L))(v)
    assert np.all(np.abs(o - right) <= 2.0 ** -8 * np.abs(right))
    assert np.mean(np.abs(o - swapped)) > 0.1


def test_down_exponent_plus_one_doubles_exactly():
    hidden, inter, E = 64, 32, 4
    blob = WL.make_experts(9, E + 1, hidden, inter)
    blob2 = blob.copy()
    eb = O.canonical_expert_size(hidden, inter)
    off = WL.expert_plane_offsets(hidden, inter)
    for xid in range(E + 1):
        s0 = xid * eb + off["down_sc"]
        blob2[s0:s0 + hidden * inter // 32] += 1
    x = WL.make_x(9, 5, hidden)
    for xid in range(E + 1):
        o1 = O.expert_forward(O.bf16_bits_to_f64(x), O.decode_expert(blob, xid, hidden, inter), 10.0)
        o2 = O.expert_forward(O.bf16_bits_to_f64(x), O.decode_expert(blob2, xid, hidden, inter), 10.0)
        assert np.array_equal(o2, 2 * o1)


# ---------------------------------------------------------------- whole layer
def _tiny_layer(T, hidden, inter, E, seed, routing="learned"):
    x = WL.make_x(seed, T, hidden)
    blob = WL.make_experts(seed, E + 1, hidden, inter)
    kw = dict(n_experts=E, hidden=hidden, inter=inter, top_k=6, route_scale=1.5, limit=10.0)
    if routing == "learned":
        w = WL.make_router(seed, hidden, E)
        return x, blob, kw, dict(w_router=w)
    table, tok = WL.make_hash(seed, T, E, 6, vocab=97)
    return x, blob, kw, dict(token_ids=tok, table=table)


@pytest.mark.parametrize("shape,routing", [((8, 64, 32, 16), "learned"), ((8, 64, 32, 16), "hash"),
                                           ((3, 512, 512, 256), "learned")])
def test_dense_brute_force_equals_sparse(shape, routing):
    T, hidden, inter, E = shape
    x, blob, kw, rk = _tiny_layer(T, hidden, inter, E, 21, routing)
    r = O.moe_layer(x, blob, **kw, **rk)
    yd = O.dense_moe_layer(x, blob, r["ids"], r["weights"], n_experts=E, hidden=hidden, inter=inter, limit=10.0)
    assert np.max(np.abs(yd - r["y"])) <= 1e-12 * np.max(np.abs(yd))
    # shapes and routing invariants
    assert r["offsets"][-1] == T * 7 and r["y"].shape == (T, hidden)
    assert np.allclose(r["weights"].sum(axis=1), 1.5, rtol=0, atol=1e-12)


def test_token_permutation_equivariance():
    T, hidden, inter, E = 12, 64, 32, 16
    x, blob, kw, rk = _tiny_layer(T, hidden, inter, E, 33)
    perm = np.random.default_rng(4).permutation(T)
    y = O.moe_layer(x, blob, **kw, **rk)["y"]
    yp = O.moe_layer(x[perm], blob, **kw, **rk)["y"]
    assert np.max(np.abs(yp - y[perm])) <= 1e-12 * np.max(np.abs(y))


def test_combine_weights_and_shared_term():
    # out rows with known values: y = sum_j w_j * row + shared row
    T, k, H = 3, 6, 4
    slot_row = np.array([[0, 1, 2, 3, 4, 5, 18], [6, 7, 8, 9, 10, 11, 19], [12, 13, 14, -1, 16, 17, 20]])
    out = np.arange(21 * H, dtype=np.float64).reshape(21, H)
    w = np.arange(T * k, dtype=np.float64).reshape(T, k) / 10
    y = O.combine(out, slot_row, w)
    for t in range(T):
        want = np.zeros(H)
        for j in range(k):
            if slot_row[t, j] >= 0:
                want += w[t, j] * out[slot_row[t, j]]
        want += out[18 + t]               # routed sum first, then the shared expert
        assert np.array_equal(y[t], want)


# ---------------------------------------------------------------- MXFP8 shared expert
def test_e4m3_table_matches_torch_float8():
    # torch's float8_e4m3fn is an independent implementation of the same OCP format
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(O.E4M3_VALUES), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(O.E4M3_VALUES[ok], t[ok])
    assert np.array_equal(np.signbit(O.E4M3_VALUES[ok]), np.signbit(t[ok]))


def test_e4m3_closed_forms():
    v = O.E4M3_VALUES
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # 1.75 * 2^8, the largest finite
    assert v[0x38] == 1.0 and v[0xB8] == -1.0               # exponent field 7 = bias
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9    # smallest normal, smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                          # largest subnormal
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])


def test_decode_mxfp8_matches_torch_and_scale_axis():
    rng = np.random.default_rng(8)
    n, k = 5, 96
    codes = rng.integers(0, 256, size=(n, k), dtype=np.int32).astype(np.uint8)
    codes[codes == 0x7F] = 0x00
    codes[codes == 0xFF] = 0x80
    scales = rng.integers(110, 135, size=(n, k // 32), dtype=np.int32).astype(np.uint8)
    w = O.decode_mxfp8(codes.ravel(), scales.ravel(), n, k)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).double()
    s = torch.from_numpy(scales.astype(np.float64) - 127.0)
    want = (t * torch.pow(2.0, s).repeat_interleave(32, dim=1)).numpy()
    assert np.array_equal(w, want)


def _mxfp8_copy_of_shared(blob, E, hidden, inter):
    """The blob with its MXFP4 shared expert re-encoded as MXFP8: each E2M1
    value is an E4M3 value too (encoded by torch), with the same scales."""
    eb = WL.expert_bytes(hidden, inter)
    off = WL.expert_plane_offsets(hidden, inter)
    base = E * eb
    e2m1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])
    to_e4m3 = e2m1.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    parts = []
    for name, n, k in (("gate", inter, hidden), ("up", inter, hidden), ("down", hidden, inter)):
        nib = blob[base + off[name + "_nib"]: base + off[name + "_nib"] + n * k // 2].reshape(n, k // 2)
        codes = np.empty((n, k), dtype=np.uint8)
        codes[:, 0::2] = to_e4m3[nib & 0x0F]      # low nibble = even column
        codes[:, 1::2] = to_e4m3[nib >> 4]
        parts += [codes.ravel(), blob[base + off[name + "_sc"]: base + off[name + "_sc"] + n * k // 32]]
    return np.concatenate([blob[:base]] + parts)


def test_mxfp8_shared_equals_its_mxfp4_original():
    # the MXFP8 reader (its own layout code) must give the layer exactly what
    # the MXFP4 reader gives for the same weights
    T, hidden, inter, E = 9, 64, 64, 16
    x, blob, kw, rk = _tiny_layer(T, hidden, inter, E, 41)
    b8 = _mxfp8_copy_of_shared(blob, E, hidden, inter)
    assert len(b8) == E * WL.expert_bytes(hidden, inter) + WL.mxfp8_expert_bytes(hidden, inter)
    assert len(b8) - E * O.canonical_expert_size(hidden, inter) == O.canonical_mxfp8_expert_size(hidden, inter)
    r4 = O.moe_layer(x, blob, **kw, **rk)
    r8 = O.moe_layer(x, b8, **kw, **rk, shared_fmt="mxfp8")
    assert np.array_equal(r4["out_rows"], r8["out_rows"]) and np.array_equal(r4["y"], r8["y"])


@pytest.mark.parametrize("routing", ["learned", "hash"])
def test_dense_brute_force_equals_sparse_mxfp8_shared(routing):
    T, hidden, inter, E = 8, 64, 32, 16
    x, _, kw, rk = _tiny_layer(T, hidden, inter, E, 23, routing)
    blob = WL.make_experts_shared_mxfp8(23, E, hidden, inter)
    r = O.moe_layer(x, blob, **kw, **rk, shared_fmt="mxfp8")
    yd = O.dense_moe_layer(x, blob, r["ids"], r["weights"], n_experts=E, hidden=hidden, inter=inter, limit=10.0,
                           shared_fmt="mxfp8")
    assert np.max(np.abs(yd - r["y"])) <= 1e-12 * np.max(np.abs(yd))
    # the format matters: the same bytes read as an MXFP4 shared expert give another y
    r4 = O.moe_layer(x, blob, **kw, **rk)
    assert np.all(np.isfinite(r["y"])) and not np.allclose(r4["y"], r["y"])


def test_mxfp8_workload_codes_and_scales():
    b = WL.make_shared_mxfp8(3, 512, 512)
    n = 512 * 512
    codes = np.concatenate([b[0:n], b[n + n // 32: 2 * n + n // 32], b[2 * (n + n // 32): 3 * n + 2 * n // 32]])
    assert not np.any((codes == 0x7F) | (codes == 0xFF))           # no NaN codes
    counts = np.bincount(codes, minlength=256)
    assert counts.min() > 0 or set(np.flatnonzero(counts == 0)) == {0x7F, 0xFF}
    sc = b[n: n + n // 32]
    assert sc.min() == 113 and sc.max() == 117


def test_top_k_equal_to_expert_count_selects_all():
    # every expert chosen, in descending key order, weights summing to 1.5; no near-tie boundary
    T, H, E = 5, 512, 7
    x = WL.make_x(3, T, H)
    w = WL.make_router(3, H, E)
    ids, wt, s = O.route_learned(x, w, None, E, 1.5)
    assert all(sorted(r) == list(range(E)) for r in ids.tolist())
    assert np.all(np.diff(np.take_along_axis(s, ids.astype(np.int64), axis=1), axis=1) <= 0)
    assert np.allclose(wt.sum(axis=1), 1.5, rtol=0, atol=1e-12)
    assert np.all(np.isinf(O.boundary_gap(x, w, None, E)))


# ---------------------------------------------------------------- 2-bit affine routed experts
def _bf16_bytes(values):
    """bf16 bytes (little-endian) of values exactly representable in bf16, via torch."""
    t = torch.tensor(values, dtype=torch.float64).to(torch.bfloat16)
    assert torch.equal(t.double(), torch.tensor(values, dtype=torch.float64))
    return t.view(torch.int16).numpy().astype("<i2").view(np.uint8)


@pytest.mark.parametrize("group", [64, 32])
def test_decode_affine2_bit_fields_and_group_axis(group):
    # codes written bit by bit in plain Python; s, b per (row, group) chosen so
    # every weight is a distinct small dyadic number, computed here in Python floats
    n, k = 3, 128
    q = [[(7 * r + c * c + c // 5) % 4 for c in range(k)] for r in range(n)]
    codes = bytearray()
    for r in range(n):
        for c0 in range(0, k, 4):
            byte = 0
            for j in range(4):
                byte |= q[r][c0 + j] << (2 * j)          # column c0+j in bits 2j+1:2j
            codes.append(byte)
    ng = k // group
    s = [[2.0 ** (r - gi) * (1 + gi / 8) for gi in range(ng)] for r in range(n)]
    b = [[-(gi + 1) * 0.25 - r for gi in range(ng)] for r in range(n)]
    w = O.decode_affine2(np.frombuffer(bytes(codes), dtype=np.uint8), _bf16_bytes(sum(s, [])),
                         _bf16_bytes(sum(b, [])), n, k, group)
    want = np.array([[s[r][c // group] * q[r][c] + b[r][c // group] for c in range(k)] for r in range(n)])
    assert np.array_equal(w, want)
    # reading the same planes with the other group size must differ (group axis pinned)
    other = 32 if group == 64 else 64
    ns = n * k // other
    alt = O.decode_affine2(np.frombuffer(bytes(codes), dtype=np.uint8), _bf16_bytes([1.0] * ns), _bf16_bytes([0.0] * ns),
                           n, k, other)
    assert np.array_equal(alt, np.array(q, dtype=np.float64))     # s = 1, b = 0 gives the codes back


def test_affine2_sizes_closed_form():
    # 2 bits per weight plus a bf16 (scale, bias) per 64 (gate, up) or 32 (down)
    # weights: (2 + 0.5) + (2 + 0.5) + (2 + 1) bits over three H*I projections = 8 bits per H*I
    for h, i in ((4096, 2048), (512, 512), (1024, 512)):
        assert O.canonical_affine2_expert_size(h, i) == h * i == WL.affine2_expert_bytes(h, i)
    assert O.AFFINE2_GROUPS == WL.AFFINE2_GROUPS == (64, 64, 32)


def _affine2_twin(E, hidden, inter, seed):
    """An affine blob and an MXFP4 blob that hold the same weights: in each
    affine group s = 2^e, b = -c 2^e (c in 0..3), so w = 2^e (q - c) is an
    integer in -3..3 times 2^e, which E2M1 codes hold exactly under the MX
    scale byte e + 127 of both 32-column halves of the group."""
    rng = np.random.default_rng(seed)
    e2m1_of_int = {0: 0x0, 1: 0x2, 2: 0x4, 3: 0x5}                  # E2M1 1.0, 2.0, 3.0
    aff, mx = [], []
    for xid in range(E):
        ab, mb = [], []
        for (n, k), gs in zip(((inter, hidden), (inter, hidden), (hidden, inter)), O.AFFINE2_GROUPS):
            q = rng.integers(0, 4, size=(n, k))
            ee = rng.integers(-8, -3, size=(n, k // gs))
            c = rng.integers(0, 4, size=(n, k // gs))
            v = q - np.repeat(c, gs, axis=1)                                 # integers -3..3
            codes = np.zeros((n, k // 4), dtype=np.uint8)
            for j in range(4):
                codes |= (q[:, j::4] << (2 * j)).astype(np.uint8)
            ab += [codes.ravel(), _bf16_bytes((2.0 ** ee).ravel().tolist()),
                   _bf16_bytes((-c * 2.0 ** ee).ravel().tolist())]
            nib = np.vectorize(lambda t: e2m1_of_int[abs(t)] | (0x8 if t < 0 else 0))(v).astype(np.uint8)
            mb += [(nib[:, 0::2] | (nib[:, 1::2] << 4)).ravel(),
                   (np.repeat(ee, gs // 32, axis=1) + 127).astype(np.uint8).ravel()]
        aff.append(np.concatenate(ab))
        mx.append(np.concatenate(mb))
    shared = WL.make_mxfp4_expert(seed, E, hidden, inter)
    return np.concatenate(aff + [shared]), np.concatenate(mx + [shared])


@pytest.mark.parametrize("routing", ["learned", "hash"])
def test_affine2_layer_equals_its_mxfp4_twin(routing):
    # the affine reader (its own layout, groups and bf16 planes) must give the
    # layer exactly what the pinned MXFP4 reader gives for the same weights
    T, hidden, inter, E = 9, 128, 64, 16
    x, _, kw, rk = _tiny_layer(T, hidden, inter, E, 43, routing)
    ba, bm = _affine2_twin(E, hidden, inter, 43)
    assert len(ba) == E * O.canonical_affine2_expert_size(hidden, inter) + O.canonical_expert_size(hidden, inter)
    ra = O.moe_layer(x, ba, **kw, **rk, routed_fmt="affine2")
    rm = O.moe_layer(x, bm, **kw, **rk)
    assert np.array_equal(ra["out_rows"], rm["out_rows"]) and np.array_equal(ra["y"], rm["y"])


@pytest.mark.parametrize("shared", ["mxfp4", "mxfp8"])
def test_dense_brute_force_equals_sparse_affine2(shared):
    T, hidden, inter, E = 8, 128, 64, 16
    x, _, kw, rk = _tiny_layer(T, hidden, inter, E, 29)
    blob = WL.make_experts_affine2(29, E, hidden, inter, shared)
    r = O.moe_layer(x, blob, **kw, **rk, routed_fmt="affine2", shared_fmt=shared)
    yd = O.dense_moe_layer(x, blob, r["ids"], r["weights"], n_experts=E, hidden=hidden, inter=inter, limit=10.0,
                           shared_fmt=shared, routed_fmt="affine2")
    assert np.max(np.abs(yd - r["y"])) <= 1e-12 * np.max(np.abs(yd))
    # the format matters: the same bytes read as MXFP4 experts give another y
    assert np.all(np.isfinite(r["y"]))
    assert not np.allclose(O.expert_forward(O.bf16_bits_to_f64(x), O.decode_expert(blob, 0, hidden, inter, "affine2",
                                                                                    "affine2"), 10.0),
                           O.expert_forward(O.bf16_bits_to_f64(x), O.decode_expert(blob, 0, hidden, inter), 10.0))


def test_affine2_workload_fields():
    hidden, inter = 512, 512
    b = WL.make_affine2_expert(3, 0, hidden, inter)
    n = inter * hidden
    codes = b[:n // 4]
    q = np.stack([(codes >> (2 * j)) & 3 for j in range(4)]).ravel()
    counts = np.bincount(q, minlength=4)
    assert counts.min() > 0.24 * q.size                              # uniform over 0..3
    sc = b[n // 4: n // 4 + 2 * (n // 64)].view("<u2")
    bi = b[n // 4 + 2 * (n // 64): n // 4 + 4 * (n // 64)].view("<u2")
    assert np.all(sc >> 15 == 0) and np.all(bi >> 15 == 1)          # scales positive, biases negative
    assert np.array_equal((sc >> 7) & 0xFF, (bi >> 7) & 0xFF)       # same exponent per group
    assert set(np.unique((sc >> 7) & 0xFF)) == set(range(119, 124))  # 2^-8 .. 2^-4
    assert np.all(sc & 0xF == 0)                                     # scale mantissa 1 + f/8
