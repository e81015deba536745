"""GPU parity of the MoE layer against the CPU oracle, through the C ABI.

Small shapes run the whole layer element by element (several tiles, ragged
tails, both expert-FFN kernel families, empty experts); the five full-size
workloads check routing and dispatch on every token and the expert rows and
outputs on sampled tokens, in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import moe_oracle as O  # noqa: E402
from mxfp4_routed_expert_moe_amd import binding as B  # noqa: E402
from mxfp4_routed_expert_moe_amd import workloads as WL  # noqa: E402
from tests import layer_check as LC  # noqa: E402

pytestmark = pytest.mark.gpu


def _small_inputs(T, hidden, inter, E, seed, routing="learned", bias=False, top_k=6):
    w = WL.Workload(90, "small", T, routing, None)
    x = WL.make_x(seed, T, hidden)
    router = b = table = tok = None
    if routing == "learned":
        router = WL.make_router(seed, hidden, E)
        if bias:
            b = (np.random.default_rng(seed).standard_normal(E) * 0.5).astype(np.float32)
    else:
        table, tok = WL.make_hash(seed, T, E, top_k, vocab=1000)
    experts = WL.make_experts(seed, E + 1, hidden, inter)
    return WL.LayerInputs(w, x, router, b, table, tok, experts, hidden, inter, E, top_k)


def _experts(inp):
    return B.Experts.from_canonical(inp.experts, inp.n_experts, inp.hidden, inp.inter)


# T*7 <= 16*(E+1) selects the decode kernels, above it the prefill kernels.
SMALL = [
    # (T, H, I, E, routing, bias)
    (1, 512, 512, 16, "learned", False),      # decode, 1 row per expert
    (5, 512, 1024, 16, "learned", False),     # decode, every group in one 16-row chunk
    (29, 1024, 512, 32, "learned", True),     # decode, selection bias
    (37, 512, 512, 16, "learned", False),     # decode, groups over 16 rows (the shared one: 3 chunks)
    (61, 512, 512, 16, "hash", False),        # hash routing
    (300, 512, 512, 16, "learned", False),    # prefill, ragged 64-row items
    (700, 512, 512, 256, "learned", False),   # prefill, 256 experts, many tiny groups
    (64, 512, 512, 256, "learned", True),     # decode with 256 experts, many empty
    (9, 512, 4096, 16, "learned", False),     # decode, down K = 4096 (eight k tiles per wave)
    (200, 2048, 4096, 16, "learned", False),  # prefill, K = 2048 and 4096
]


@pytest.mark.parametrize("T,H,I,E,routing,bias", SMALL)
def test_layer_small_shapes(T, H, I, E, routing, bias):
    print(f"[parity] small T={T} H={H} I={I} E={E} {routing} bias={bias}", flush=True)
    inp = _small_inputs(T, H, I, E, 1000 + T, routing, bias)
    r = LC.full_check(inp, _experts(inp))
    assert r["ambiguous"] == 0
    # every row, not just a sample: compare all expert rows too
    g = r["g"]
    ref = O.moe_layer(inp.x, inp.experts, n_experts=E, hidden=H, inter=I, top_k=6, route_scale=1.5,
                      limit=WL.CLAMP_LIMIT, w_router=inp.router, bias=inp.bias, token_ids=inp.tok, table=inp.table)
    n = int(ref["offsets"][-1])
    LC.assert_output_close(LC.host(g["out_rows"][:n]), ref["out_rows"], "all rows")
    LC.assert_output_close(O.bf16_bits_to_f64(g["y"]), ref["y"], "all outputs")


@pytest.mark.parametrize("T,E,top_k,routing", [
    (20, 100, 1, "learned"),    # one expert per token, E not a multiple of 64 (or of 16)
    (20, 100, 8, "learned"),    # the largest top_k
    (150, 48, 8, "learned"),    # prefill kernels (T*(k+1) > 16*(E+1)), largest top_k
    (400, 48, 1, "hash"),       # prefill kernels with one routed row per token
])
def test_top_k_and_expert_count_extremes(T, E, top_k, routing):
    print(f"[parity] top_k={top_k} E={E} T={T} {routing}", flush=True)
    inp = _small_inputs(T, 512, 512, E, 7000 + T + top_k, routing, top_k=top_k)
    r = LC.full_check(inp, _experts(inp))
    assert r["ambiguous"] == 0
    g = r["g"]
    ref = O.moe_layer(inp.x, inp.experts, n_experts=E, hidden=512, inter=512, top_k=top_k, route_scale=1.5,
                      limit=WL.CLAMP_LIMIT, w_router=inp.router, bias=inp.bias, token_ids=inp.tok, table=inp.table)
    LC.assert_output_close(O.bf16_bits_to_f64(g["y"]), ref["y"], "all outputs")


@pytest.mark.parametrize("T", [6, 300])   # decode and prefill kernels
def test_wide_scale_range(T):
    # E8M0 scales over 2^-27 .. 2^13: exercises the scale operand of the
    # convert across exponents and saturates the clamp on most rows
    H, I, E = 512, 512, 16
    inp = _small_inputs(T, H, I, E, 4242)
    inp.experts = WL.make_experts(4242, E + 1, H, I, scale_lo=100, scale_hi=140)
    r = LC.full_check(inp, _experts(inp))
    assert r["ambiguous"] == 0


def test_determinism_bitwise():
    inp = _small_inputs(300, 512, 512, 16, 77)
    ex = _experts(inp)
    a = LC.run_gpu_layer(inp, ex)
    b = LC.run_gpu_layer(inp, ex)
    assert np.array_equal(a["y"], b["y"])
    assert torch.equal(a["out_rows"], b["out_rows"])
    inp2 = _small_inputs(40, 512, 512, 16, 78)
    ex2 = _experts(inp2)
    assert np.array_equal(LC.run_gpu_layer(inp2, ex2)["y"], LC.run_gpu_layer(inp2, ex2)["y"])
    # mostly full items (T * k >= 128 E): the prefill instance whose blocks
    # take two column blocks in turn
    inp3 = _small_inputs(2000, 512, 512, 16, 79)
    ex3 = _experts(inp3)
    c = LC.run_gpu_layer(inp3, ex3)
    d = LC.run_gpu_layer(inp3, ex3)
    assert np.array_equal(c["y"], d["y"])
    assert torch.equal(c["out_rows"], d["out_rows"])


@pytest.mark.parametrize("T", [3, 200])
def test_down_exponent_plus_one_doubles_bitwise(T):
    # a power-of-two rescale of every down weight doubles each expert row exactly
    inp = _small_inputs(T, 512, 512, 16, 55)
    ex1 = _experts(inp)
    blob2 = inp.experts.copy()
    eb = WL.expert_bytes(512, 512)
    off = WL.expert_plane_offsets(512, 512)
    for xid in range(17):
        s0 = xid * eb + off["down_sc"]
        blob2[s0:s0 + 512 * 512 // 32] += 1
    ex2 = B.Experts.from_canonical(blob2, 16, 512, 512)
    a = LC.run_gpu_layer(inp, ex1)
    b = LC.run_gpu_layer(inp, ex2)
    n = int(a["offsets"][-1])
    assert torch.equal(b["out_rows"][:n], 2 * a["out_rows"][:n])


def _identity_blob(hidden, inter, n_total, up_code):
    eb = WL.expert_bytes(hidden, inter)
    off = WL.expert_plane_offsets(hidden, inter)
    blob = np.zeros(n_total * eb, dtype=np.uint8)
    for xid in range(n_total):
        b = xid * eb
        for name, code in (("gate", 0x2), ("up", up_code)):
            nib = blob[b + off[name + "_nib"]: b + off[name + "_nib"] + inter * hidden // 2].reshape(inter, hidden // 2)
            i = np.arange(inter)
            nib[i, i // 2] |= (code << (4 * (i & 1))).astype(np.uint8)
            blob[b + off[name + "_sc"]: b + off[name + "_sc"] + inter * hidden // 32] = 127
        nib = blob[b + off["down_nib"]: b + off["down_nib"] + hidden * inter // 2].reshape(hidden, inter // 2)
        i = np.arange(inter)
        nib[i, i // 2] |= (0x2 << (4 * (i & 1))).astype(np.uint8)
        blob[b + off["down_sc"]: b + off["down_sc"] + hidden * inter // 32] = 127
    return blob


@pytest.mark.parametrize("T,split", [(4, False), (300, False), (300, True)])
def test_identity_experts_closed_form_and_orientation(T, split):
    # gate = I, up = 2I, down = I: every expert row is silu(min(x,L)) * clamp(2x,-L,L)
    # in its first I columns and 0 beyond; a swapped gate/up would differ.
    H, I, E, L = 1024, 512, 16, WL.CLAMP_LIMIT
    inp = _small_inputs(T, H, I, E, 91)
    xf = np.random.default_rng(5).standard_normal((T, H)).astype(np.float32) * 4
    xf[0, :6] = [12.0, -12.0, 9.99, -9.99, 10.0, -10.0]
    inp.x = WL.f32_to_bf16_bits(xf)
    blob = _identity_blob(H, I, E + 1, 0x4)
    inp.experts = blob
    g = LC.run_gpu_layer(inp, B.Experts.from_canonical(blob, E, H, I, split_fp8=split))
    rows = LC.host(g["out_rows"][: int(g["offsets"][-1])]).astype(np.float64)
    v = O.bf16_bits_to_f64(inp.x)[g["row_token"][: rows.shape[0]], :I]
    silu = lambda a: a / (1 + np.exp(-a))  # noqa: E731
    want = silu(np.minimum(v, L)) * np.clip(2 * v, -L, L)
    # h is rounded to bf16 (half an ulp: 2^-8 relative); the fp32 SiLU adds ~1e-6.
    tol = 2.0 ** -8 * (1 + 1e-4) * np.abs(want) + 1e-30
    if split:
        # Two E4M3 terms under one power-of-two scale per 32 k are exact down
        # to 2^-13 of the block's largest magnitude and off by at most 2^-21
        # of it below that.  For x this moves only |v| < 2^-13 max|x|, where
        # the SwiGLU slope is about 2|v|; for h it lands on the output as is
        # (identity down weights, one product per output): 2^-21 of the
        # 32-column block maximum.
        blk = np.repeat(np.abs(want).reshape(want.shape[0], I // 32, 32).max(axis=2), 32, axis=1)
        tol = tol + 2.0 ** -21 * blk
        # the expert row is rounded to bf16 once more (half an ulp, 2^-9
        # relative), no longer exactly h once the split has moved it
        tol = tol + 2.0 ** -9 * np.abs(rows[:, :I])
    assert np.all(np.abs(rows[:, :I] - want) <= tol)
    assert np.all(rows[:, I:] == 0)
    swapped = silu(np.minimum(2 * v, L)) * np.clip(v, -L, L)
    assert np.mean(np.abs(rows[:, :I] - swapped)) > 0.1


def test_edge_cases_empty_and_dropped_ids():
    H, I, E = 512, 512, 16
    inp = _small_inputs(9, H, I, E, 12)
    ex = _experts(inp)
    layer = B.MoeLayer(ex, 9, 6, 1.5, WL.CLAMP_LIMIT, w_router=LC.dev(inp.router))
    # T = 0 is a no-op through every call
    assert B.lib().moe_combine(None, None, None, 0, H, 6, None, None) == 0
    # dispatch + ffn + combine with ids containing out-of-range values: they are dropped
    ids = np.stack([np.random.default_rng(i).permutation(E)[:6] for i in range(9)]).astype(np.int32)
    ids[2, 1] = E + 5
    ids[4, 0] = -7
    layer.ids.copy_(LC.dev(ids))
    layer.weights.fill_(0.25)
    layer.dispatch()
    xd = LC.dev(inp.x)
    layer.expert_ffn(xd)
    layer.combine()
    torch.cuda.synchronize()
    off, rt, sr = O.dispatch(ids, E)
    assert np.array_equal(LC.host(layer.offsets), off)
    assert np.array_equal(LC.host(layer.slot_row), sr)
    assert np.array_equal(LC.host(layer.row_token)[: off[-1]], rt)
    out = O.expert_ffn(inp.x, inp.experts, off, rt, WL.CLAMP_LIMIT, E, H, I)
    y = O.combine(out, sr, np.full((9, 6), 0.25))
    LC.assert_output_close(O.bf16_bits_to_f64(LC.host(layer.y).view(np.uint16)), y, "dropped ids")


@pytest.mark.parametrize("T", [50, 400])   # single-block dispatch (T*6 <= 2048) and the chunked path
def test_dispatch_duplicates_and_invalid_ids(T):
    E = 40
    g = np.random.default_rng(T)
    ids = g.integers(0, E, size=(T, 6)).astype(np.int32)      # repeats inside a token are allowed
    ids[g.integers(0, T, 7), g.integers(0, 6, 7)] = E + 1       # dropped
    ids[g.integers(0, T, 5), g.integers(0, 6, 5)] = -3          # dropped
    off, rt, sr = B.dispatch(LC.dev(ids), E)
    o2, r2, s2 = O.dispatch(ids, E)
    assert np.array_equal(LC.host(off), o2)
    assert np.array_equal(LC.host(rt)[: o2[-1]], r2)
    assert np.array_equal(LC.host(sr), s2)


@pytest.mark.parametrize("T", [20, 300])
def test_ffn_phases_equal_one_call(T):
    inp = _small_inputs(T, 512, 512, 16, 66)
    ex = _experts(inp)
    a = LC.run_gpu_layer(inp, ex)
    layer = a["layer"]
    ref = layer.out_rows.clone()
    layer.out_rows.zero_()
    xd = LC.dev(inp.x)
    for ph in (0, 1, 2):
        layer.expert_ffn_phase(xd, ph)
    torch.cuda.synchronize()
    n = int(a["offsets"][-1])
    assert torch.equal(layer.out_rows[:n], ref[:n])


# Learned routing on each logits path: up to 256 tokens take the float64
# vector-unit kernel; more tokens with 16-byte aligned router weights (E a
# multiple of 64) take the bf16 matrix-core split path with its bound and
# float64 list, and the same weights 4 bytes off that alignment the vector-unit
# kernel.  All must give the oracle's ids bit for bit and its weights, and
# each other's ids.
ROUTER_SHAPES = [
    # (T, H, E, bias)
    (3, 512, 16, False),       # a ragged 8-token block, few experts
    (40, 1024, 64, True),
    (200, 4096, 256, False),   # full hidden size and expert count, few tokens
    (257, 512, 64, True),      # one token past the many-token threshold, ragged 32-token blocks
    (300, 1024, 128, False),
    (1000, 4096, 256, True),   # full hidden size and expert count
    (600, 1536, 192, True),    # six waves per split-logits block, three k stages per slice
]


@pytest.mark.parametrize("T,H,E,bias", ROUTER_SHAPES)
def test_router_kernels_many_tokens(T, H, E, bias):
    print(f"[parity] router T={T} H={H} E={E} bias={bias}", flush=True)
    seed = 3000 + T
    x = WL.make_x(seed, T, H)
    router = WL.make_router(seed, H, E)
    b = (np.random.default_rng(seed).standard_normal(E) * 0.5).astype(np.float32) if bias else None
    ids_ref, w_ref, _ = O.route_learned(x, router, b, 6, WL.ROUTE_SCALE)
    gap = O.boundary_gap(x, router, b, 6)
    xd = LC.dev(x)
    bd = None if b is None else LC.dev(b)
    aligned = LC.dev(router.reshape(-1))
    assert aligned.data_ptr() % 16 == 0
    off = torch.empty(H * E + 1, dtype=torch.float32, device="cuda")
    off[1:] = aligned
    shifted = off[1:]
    assert shifted.data_ptr() % 16 == 4
    got = {}
    for name, w in (("aligned", aligned), ("vector", shifted)):
        ids, wts = B.route(xd, T, E, 6, WL.ROUTE_SCALE, w_router=w, sel_bias=bd)
        torch.cuda.synchronize()
        got[name] = dict(ids=LC.host(ids), weights=LC.host(wts))
        LC.check_routing(got[name], ids_ref, w_ref, gap)
        # the six weights of a token sum to the route scale (float32 weights, summed exactly)
        wsum = got[name]["weights"].astype(np.float64).sum(axis=1)
        assert np.max(np.abs(wsum - WL.ROUTE_SCALE)) <= 4 * np.spacing(np.float32(WL.ROUTE_SCALE))
    clear = gap >= LC.AMBIGUOUS_GAP
    assert np.array_equal(got["aligned"]["ids"][clear], got["vector"]["ids"][clear])


@pytest.mark.parametrize("T", [40, 300])   # decode-size and many-token logits kernels
def test_router_exact_ties_go_to_the_lower_id(T):
    """Three router columns made identical (and large) give three equal keys
    inside the top 6 for about half of the tokens; the ids must come out in
    ascending order among them, as the oracle orders equal keys."""
    print(f"[parity] router ties T={T}", flush=True)
    H, E = 512, 256
    seed = 4000 + T
    x = WL.make_x(seed, T, H)
    router = WL.make_router(seed, H, E)
    router[:, 7] *= 10.0
    router[:, 130] = router[:, 7]
    router[:, 201] = router[:, 7]
    ids_ref, w_ref, _ = O.route_learned(x, router, None, 6, WL.ROUTE_SCALE)
    gap = O.boundary_gap(x, router, None, 6)
    ids, wts = B.route(LC.dev(x), T, E, 6, WL.ROUTE_SCALE, w_router=LC.dev(router))
    torch.cuda.synchronize()
    g = dict(ids=LC.host(ids), weights=LC.host(wts))
    LC.check_routing(g, ids_ref, w_ref, gap)
    tied = (ids_ref[:, :3] == np.array([7, 130, 201])).all(axis=1)
    assert tied.sum() >= T // 4, "the tie case did not occur often enough to test it"  # 15 of 40, 113 of 300
    assert (g["ids"][tied, :3] == np.array([7, 130, 201])).all()


@pytest.mark.parametrize("T", [24, 300])   # decode-size and many-token logits kernels
def test_forced_routing_by_bias(T):
    """A +1e6 selection bias on six chosen experts selects exactly those for
    every token, ordered by their unbiased scores, with weights from the
    unbiased scores."""
    print(f"[parity] forced routing T={T}", flush=True)
    H, E = 1024, 256
    seed = 6000 + T
    x = WL.make_x(seed, T, H)
    router = WL.make_router(seed, H, E)
    chosen = np.array([3, 77, 100, 101, 200, 255])
    b = np.zeros(E, dtype=np.float32)
    b[chosen] = 1e6
    ids_ref, w_ref, _ = O.route_learned(x, router, b, 6, WL.ROUTE_SCALE)
    gap = O.boundary_gap(x, router, b, 6)
    assert (np.sort(ids_ref, axis=1) == chosen).all()
    ids, wts = B.route(LC.dev(x), T, E, 6, WL.ROUTE_SCALE, w_router=LC.dev(router), sel_bias=LC.dev(b))
    torch.cuda.synchronize()
    g = dict(ids=LC.host(ids), weights=LC.host(wts))
    assert (np.sort(g["ids"], axis=1) == chosen).all()
    LC.check_routing(g, ids_ref, w_ref, gap)


@pytest.mark.parametrize("T", [300, 5000, 20000])   # 20000: 10000 listed tokens, two h slices per listed block
def test_router_zero_rows_go_to_the_float64_list(T):
    """Every other token's x row is zero: all its logits are 0, its keys tie,
    and the matrix-core bound cannot order them, so those tokens (half the
    batch) are decided on the float64 list: ids 0..5 in order, equal weights.
    The other tokens are decided as usual."""
    print(f"[parity] router zero rows T={T}", flush=True)
    H, E = 1024, 256
    seed = 7000 + T
    x = WL.make_x(seed, T, H)
    x[1::2] = 0
    router = WL.make_router(seed, H, E)
    ids_ref, w_ref, _ = O.route_learned(x, router, None, 6, WL.ROUTE_SCALE)
    gap = O.boundary_gap(x, router, None, 6)
    ids, wts = B.route(LC.dev(x), T, E, 6, WL.ROUTE_SCALE, w_router=LC.dev(router))
    torch.cuda.synchronize()
    g = dict(ids=LC.host(ids), weights=LC.host(wts))
    z = slice(1, None, 2)
    assert (ids_ref[z] == np.arange(6)).all()
    assert np.array_equal(g["ids"][z], ids_ref[z])
    assert np.array_equal(g["weights"][z], w_ref[z].astype(np.float32))
    live = np.arange(0, T, 2)
    sub = dict(ids=g["ids"][live], weights=g["weights"][live])
    LC.check_routing(sub, ids_ref[live], w_ref[live], gap[live])


def test_router_huge_weight_sends_every_token_to_the_float64_list():
    """A router weight of 2^121 fails the split's range check, so every
    token's selection comes from the float64 logits; the result must still be
    the oracle's."""
    print("[parity] router huge weight", flush=True)
    T, H, E = 700, 1024, 256
    seed = 7500
    x = WL.make_x(seed, T, H)
    router = WL.make_router(seed, H, E)
    router[5, 17] = np.float32(2.0 ** 121)
    ids_ref, w_ref, _ = O.route_learned(x, router, None, 6, WL.ROUTE_SCALE)
    gap = O.boundary_gap(x, router, None, 6)
    ids, wts = B.route(LC.dev(x), T, E, 6, WL.ROUTE_SCALE, w_router=LC.dev(router))
    torch.cuda.synchronize()
    g = dict(ids=LC.host(ids), weights=LC.host(wts))
    LC.check_routing(g, ids_ref, w_ref, gap)
    assert (g["ids"][:, 0] == 17).sum() > T // 3


def test_hash_out_of_range_token_gives_dropped_ids():
    E = 16
    table, tok = WL.make_hash(3, 10, E, 6, vocab=50)
    tok[3] = 50
    tok[7] = -1
    ids, w = B.route(None, 10, E, 6, 1.5, token_ids=LC.dev(tok), hash_table=LC.dev(table))
    ids = LC.host(ids)
    assert np.all(ids[3] == -1) and np.all(ids[7] == -1)
    ok = [t for t in range(10) if t not in (3, 7)]
    assert np.array_equal(ids[ok], table[tok[ok]])
    assert np.all(LC.host(w) == 0.25)


# ---------------------------------------------------------------- full-size workloads
_EXPERTS_CACHE = {}


def _full_inputs(index):
    w = WL.WORKLOADS[index]
    if w.seed not in _EXPERTS_CACHE:
        _EXPERTS_CACHE.clear()
        canon = WL.make_experts(w.seed, WL.N_EXPERTS + 1)
        _EXPERTS_CACHE[w.seed] = (canon, B.Experts.from_canonical(canon, WL.N_EXPERTS, WL.HIDDEN, WL.INTER))
    canon, ex = _EXPERTS_CACHE[w.seed]
    return WL.make_layer_inputs(w, experts=canon), ex


# Every full-size workload: routing on every token (bit-exact ids, no token
# excused as a near tie), dispatch on every pair, every row and output written
# (NaN-filled beforehand), whole experts against the oracle (the hottest, the
# shared one, the smallest and eight whose row count is not a multiple of 64),
# y of every token against the oracle's combine of the GPU's rows, and the
# sampled tokens end to end.
@pytest.mark.parametrize("index,sample", [(0, None), (1, 12), (2, 12), (3, 8), (4, 8)])
def test_full_workloads(index, sample):
    w = WL.WORKLOADS[index]
    print(f"[parity] full workload {w.name} T={w.T}", flush=True)
    inp, ex = _full_inputs(index)
    r = LC.full_check(inp, ex, sample_tokens=sample, seed=index, whole=8, y_all=True)
    print(f"[parity] {w.name}: rows max/mean rel {r['rows_err'][0]:.2e}/{r['rows_err'][1]:.2e}, "
          f"y max/mean rel {r['y_err'][0]:.2e}/{r['y_err'][1]:.2e}, whole experts {r['whole_groups']} "
          f"max/mean {r['whole_err'][0]:.2e}/{r['whole_err'][1]:.2e}, combine of all tokens "
          f"{r['combine_err'][0]:.2e}/{r['combine_err'][1]:.2e}, ambiguous {r['ambiguous']}", flush=True)
    assert r["ambiguous"] == 0
    if index == 4:
        counts = np.diff(r["g"]["offsets"][: WL.N_EXPERTS + 1])
        assert counts.max() >= 0.98 * w.T              # the hottest expert takes nearly every token
        assert np.median(counts) < 200
    del r
    torch.cuda.empty_cache()


# The largest batch the boundary accepts: MOE_MAX_TOKENS tokens on the
# Zipf-skewed router of the 16384-token workload (the hottest expert takes
# nearly every token, 4096 items of 64 rows), for the default prefill path,
# the scaled-FP4 option and 2-bit affine routed experts.  7 * 262144 rows of
# H = 4096 put most element offsets into out_rows, h and the activations past
# 2^31.  Routing is checked on 1024 random tokens plus the first and the last,
# dispatch on every pair, every row and output for being written (NaN-filled
# beforehand), expert rows and outputs on 4 tokens, and every row of the
# smallest expert and of four with a ragged last item.
@pytest.mark.parametrize("path", ["mxfp4", "split_fp8", "affine2"])
def test_max_tokens(path):
    w = WL.WORKLOADS[4]
    T = B.MOE_MAX_TOKENS
    print(f"[parity] {w.name} router at T={T}, {path}", flush=True)
    routed_fmt = "mxfp4"
    if path == "affine2":
        _EXPERTS_CACHE.clear()
        canon = WL.make_experts_affine2(w.seed, WL.N_EXPERTS)
        ex = B.Experts.from_canonical(canon, WL.N_EXPERTS, WL.HIDDEN, WL.INTER, routed_affine2=True)
        routed_fmt = "affine2"
    else:
        _, ex = _full_inputs(4)
        canon = _EXPERTS_CACHE[w.seed][0]
        if path == "split_fp8":
            ex = B.Experts(ex.blob, WL.N_EXPERTS, WL.HIDDEN, WL.INTER, split_fp8=True)
    inp = WL.make_layer_inputs(w, T=T, experts=canon)
    r = LC.full_check(inp, ex, sample_tokens=4, seed=7, route_sample=1024, routed_fmt=routed_fmt, whole=4,
                      whole_big=False)
    assert r["ambiguous"] == 0
    off = r["g"]["offsets"]
    assert int(off[-1]) > (1 << 31) // WL.HIDDEN             # rows whose element offsets pass 2^31
    assert np.diff(off[: WL.N_EXPERTS + 1]).max() >= 0.98 * T
    sr = r["g"]["slot_row"][r["tokens"]]
    assert len(r["tokens"]) > 0 and (int(sr.max()) + 1) * WL.HIDDEN > 1 << 31   # checked rows past 2^31
    print(f"[parity] T={T} {path}: rows max/mean rel {r['rows_err'][0]:.2e}/{r['rows_err'][1]:.2e}, "
          f"y max/mean rel {r['y_err'][0]:.2e}/{r['y_err'][1]:.2e}", flush=True)
    del r, inp, ex
    torch.cuda.empty_cache()


# Activations of more than 4 GiB (T * H * 2 = 2^32: MOE_MAX_TOKENS tokens of
# H = 8192): the MXFP4 gate/up launch then gathers its token rows by 64-bit
# address instead of a 32-bit buffer offset.  Hash routing over 16 experts with
# I = 512 keeps the experts small; every row and output is checked for being
# written, expert rows and outputs on 6 tokens (at least one past 2^31 bytes
# into x).
def test_gateup_activations_beyond_4gib():
    T, H, I, E = B.MOE_MAX_TOKENS, 8192, 512, 16
    assert T * H * 2 >= 1 << 32
    print(f"[parity] activations beyond 4 GiB: T={T} H={H} I={I} E={E}", flush=True)
    inp = _small_inputs(T, H, I, E, 4242, routing="hash")
    r = LC.full_check(inp, _experts(inp), sample_tokens=6, seed=13, route_sample=1024)
    assert r["ambiguous"] == 0
    assert len(r["tokens"]) > 0 and int(np.max(r["tokens"])) * H * 2 >= 1 << 31
    print(f"[parity] T={T} H={H}: rows max/mean rel {r['rows_err'][0]:.2e}/{r['rows_err'][1]:.2e}, "
          f"y max/mean rel {r['y_err'][0]:.2e}/{r['y_err'][1]:.2e}", flush=True)
    del r, inp
    torch.cuda.empty_cache()


# The prefill expert FFN on the scaled FP4 matrix cores (MOE_FFN_SPLIT_FP8).
@pytest.mark.parametrize("T,H,I,E", [(300, 512, 512, 16), (700, 512, 512, 256), (200, 1024, 2048, 32)])
def test_split_fp8_small_shapes(T, H, I, E):
    print(f"[parity] split fp8 T={T} H={H} I={I} E={E}", flush=True)
    inp = _small_inputs(T, H, I, E, 1000 + T)
    ex = B.Experts.from_canonical(inp.experts, E, H, I, split_fp8=True)
    r = LC.full_check(inp, ex)
    assert r["ambiguous"] == 0
    g = r["g"]
    ref = O.moe_layer(inp.x, inp.experts, n_experts=E, hidden=H, inter=I, top_k=6, route_scale=1.5,
                      limit=WL.CLAMP_LIMIT, w_router=inp.router, bias=inp.bias, token_ids=inp.tok, table=inp.table)
    assert np.array_equal(g["offsets"], ref["offsets"])
    n = int(ref["offsets"][-1])
    LC.assert_output_close(LC.host(g["out_rows"][:n]), ref["out_rows"], "all rows")
    LC.assert_output_close(O.bf16_bits_to_f64(g["y"]), ref["y"], "all outputs")


def test_split_fp8_leaves_decode_unchanged():
    # the flag moves only the prefill family: decode-sized calls are bit-identical
    inp = _small_inputs(6, 1024, 512, 32, 77)
    a = LC.run_gpu_layer(inp, _experts(inp))
    b = LC.run_gpu_layer(inp, B.Experts.from_canonical(inp.experts, 32, 1024, 512, split_fp8=True))
    n = int(a["offsets"][-1])
    assert torch.equal(a["out_rows"][:n], b["out_rows"][:n])


@pytest.mark.parametrize("index,sample", [(3, 8), (4, 8)])
def test_split_fp8_full_prefill_workloads(index, sample):
    w = WL.WORKLOADS[index]
    print(f"[parity] split fp8 full workload {w.name} T={w.T}", flush=True)
    inp, _ = _full_inputs(index)
    ex = B.Experts(_full_inputs(index)[1].blob, WL.N_EXPERTS, WL.HIDDEN, WL.INTER, split_fp8=True)
    r = LC.full_check(inp, ex, sample_tokens=sample, seed=index, whole=4, y_all=True)
    assert r["ambiguous"] == 0
    print(f"[parity] split fp8 {w.name}: rows max/mean rel {r['rows_err'][0]:.2e}/{r['rows_err'][1]:.2e}, "
          f"y max/mean rel {r['y_err'][0]:.2e}/{r['y_err'][1]:.2e}", flush=True)
    del r
    torch.cuda.empty_cache()


# The shared expert in MXFP8 (MOE_SHARED_MXFP8).
def _shared8_inputs(T, H, I, E, seed, routing="learned"):
    inp = _small_inputs(T, H, I, E, seed, routing)
    inp.experts = WL.make_experts_shared_mxfp8(seed, E, H, I)
    return inp


@pytest.mark.parametrize("T,H,I,E,routing", [
    (5, 512, 1024, 16, "learned"),     # decode, one chunk of the shared group
    (37, 512, 512, 16, "learned"),     # decode, the shared group spans 3 chunks
    (61, 1024, 512, 64, "hash"),       # decode, hash routing
    (300, 512, 512, 16, "learned"),    # prefill, ragged 64-row items
    (200, 1024, 2048, 32, "learned"),  # prefill, K = 1024 and 2048
])
def test_shared_mxfp8_small_shapes(T, H, I, E, routing):
    print(f"[parity] shared mxfp8 T={T} H={H} I={I} E={E} {routing}", flush=True)
    inp = _shared8_inputs(T, H, I, E, 1000 + T, routing)
    ex = B.Experts.from_canonical(inp.experts, E, H, I, shared_mxfp8=True)
    r = LC.full_check(inp, ex, shared_fmt="mxfp8")
    assert r["ambiguous"] == 0
    g = r["g"]
    ref = O.moe_layer(inp.x, inp.experts, n_experts=E, hidden=H, inter=I, top_k=6, route_scale=1.5,
                      limit=WL.CLAMP_LIMIT, w_router=inp.router, bias=inp.bias, token_ids=inp.tok, table=inp.table,
                      shared_fmt="mxfp8")
    n = int(ref["offsets"][-1])
    LC.assert_output_close(LC.host(g["out_rows"][:n]), ref["out_rows"], "all rows")
    LC.assert_output_close(O.bf16_bits_to_f64(g["y"]), ref["y"], "all outputs")


def _mxfp8_reencode_shared(blob, E, H, I):
    """The MXFP4 shared expert re-encoded as MXFP8 (same values, same scales)."""
    eb = WL.expert_bytes(H, I)
    off = WL.expert_plane_offsets(H, I)
    e2m1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])
    code8 = e2m1.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    parts = [blob[:E * eb]]
    for name, n, k in (("gate", I, H), ("up", I, H), ("down", H, I)):
        nib = blob[E * eb + off[name + "_nib"]: E * eb + off[name + "_nib"] + n * k // 2].reshape(n, k // 2)
        codes = np.empty((n, k), dtype=np.uint8)
        codes[:, 0::2] = code8[nib & 0x0F]
        codes[:, 1::2] = code8[nib >> 4]
        parts += [codes.ravel(), blob[E * eb + off[name + "_sc"]: E * eb + off[name + "_sc"] + n * k // 32]]
    return np.concatenate(parts)


# decode; prefill; prefill with a shared-expert grid of 4 x 5 blocks (fewer
# than 8 * ceil(20 / 8): the block order's coverage needs the grid slack)
@pytest.mark.parametrize("T,H", [(37, 1024), (300, 1024), (300, 512)])
def test_shared_mxfp8_reencoding_is_bit_identical(T, H):
    # the same weights as MXFP4 and as MXFP8 decode to the same bf16 values and
    # are summed in the same order, so the layer must not change by one bit
    I, E = 512, 16
    inp = _small_inputs(T, H, I, E, 500 + T)
    a = LC.run_gpu_layer(inp, _experts(inp))
    b8 = _mxfp8_reencode_shared(inp.experts, E, H, I)
    b = LC.run_gpu_layer(inp, B.Experts.from_canonical(b8, E, H, I, shared_mxfp8=True))
    n = int(a["offsets"][-1])
    assert torch.equal(a["out_rows"][:n], b["out_rows"][:n]) and np.array_equal(a["y"], b["y"])


@pytest.mark.parametrize("index,sample", [(1, 12), (3, 8)])
def test_shared_mxfp8_full_workloads(index, sample):
    w = WL.WORKLOADS[index]
    print(f"[parity] shared mxfp8 full workload {w.name} T={w.T}", flush=True)
    _EXPERTS_CACHE.clear()
    canon = WL.make_experts_shared_mxfp8(w.seed, WL.N_EXPERTS)
    inp = WL.make_layer_inputs(w, experts=canon)
    ex = B.Experts.from_canonical(canon, WL.N_EXPERTS, WL.HIDDEN, WL.INTER, shared_mxfp8=True)
    r = LC.full_check(inp, ex, sample_tokens=sample, seed=index, shared_fmt="mxfp8", whole=4, y_all=True)
    assert r["ambiguous"] == 0
    print(f"[parity] shared mxfp8 {w.name}: rows max/mean rel {r['rows_err'][0]:.2e}/{r['rows_err'][1]:.2e}, "
          f"y max/mean rel {r['y_err'][0]:.2e}/{r['y_err'][1]:.2e}", flush=True)
    del r, ex
    torch.cuda.empty_cache()


# The routed experts in the 2-bit affine codec (MOE_ROUTED_AFFINE2): both
# kernel families; an MXFP4 shared expert rides in the decode launch and has
# its own prefill launch, an MXFP8 one has its own launches.
def _affine2_inputs(T, H, I, E, seed, routing="learned", shared="mxfp4"):
    inp = _small_inputs(T, H, I, E, seed, routing)
    inp.experts = WL.make_experts_affine2(seed, E, H, I, shared)
    return inp


@pytest.mark.parametrize("T,H,I,E,routing,shared", [
    (5, 512, 1024, 16, "learned", "mxfp4"),     # one chunk per group
    (37, 512, 512, 16, "learned", "mxfp4"),     # routed groups and the shared group over 16 rows: several chunks
    (61, 1024, 512, 64, "hash", "mxfp4"),       # hash routing; gate/up K = 1024
    (300, 512, 512, 16, "learned", "mxfp4"),    # prefill family, ragged 64-row items (~112 rows per expert)
    (200, 1024, 2048, 32, "learned", "mxfp4"),  # prefill family, gate/up K = 1024 (groups of 64), down K = 2048 (32)
    (40, 512, 2048, 64, "learned", "mxfp4"),    # decode family, down K = 2048 (four k tiles per wave, two-deep ring)
    (37, 512, 512, 16, "learned", "mxfp8"),     # with the MXFP8 shared expert (the recipe's 8-bit shared expert)
    (9, 4096, 512, 16, "learned", "mxfp8"),     # gate/up K = 4096 (eight k tiles per wave)
    (9, 512, 4096, 16, "learned", "mxfp4"),     # down K = 4096 (eight k tiles per wave)
    (200, 2048, 4096, 16, "learned", "mxfp4"),  # prefill family, K = 2048 and 4096
])
def test_affine2_small_shapes(T, H, I, E, routing, shared):
    print(f"[parity] affine2 T={T} H={H} I={I} E={E} {routing} shared {shared}", flush=True)
    inp = _affine2_inputs(T, H, I, E, 2000 + T, routing, shared)
    ex = B.Experts.from_canonical(inp.experts, E, H, I, shared_mxfp8=shared == "mxfp8", routed_affine2=True)
    r = LC.full_check(inp, ex, shared_fmt=shared, routed_fmt="affine2")
    assert r["ambiguous"] == 0
    g = r["g"]
    ref = O.moe_layer(inp.x, inp.experts, n_experts=E, hidden=H, inter=I, top_k=6, route_scale=1.5,
                      limit=WL.CLAMP_LIMIT, w_router=inp.router, bias=inp.bias, token_ids=inp.tok, table=inp.table,
                      shared_fmt=shared, routed_fmt="affine2")
    n = int(ref["offsets"][-1])
    LC.assert_output_close(LC.host(g["out_rows"][:n]), ref["out_rows"], "all rows")
    LC.assert_output_close(O.bf16_bits_to_f64(g["y"]), ref["y"], "all outputs")
    print(f"[parity] affine2 T={T}: rows max/mean rel {r['rows_err'][0]:.2e}/{r['rows_err'][1]:.2e}", flush=True)


def test_affine2_deterministic_and_phases():
    # two runs bit-identical; the three FFN phases one at a time equal one call
    T, H, I, E = 37, 512, 512, 16
    inp = _affine2_inputs(T, H, I, E, 77)
    ex = B.Experts.from_canonical(inp.experts, E, H, I, routed_affine2=True)
    a = LC.run_gpu_layer(inp, ex)
    b = LC.run_gpu_layer(inp, ex)
    n = int(a["offsets"][-1])
    assert torch.equal(a["out_rows"][:n], b["out_rows"][:n]) and np.array_equal(a["y"], b["y"])
    layer = a["layer"]
    ref = layer.out_rows.clone()
    layer.out_rows.zero_()
    xd = LC.dev(inp.x)
    for ph in (0, 1, 2):
        layer.expert_ffn_phase(xd, ph)
    torch.cuda.synchronize()
    assert torch.equal(layer.out_rows[:n], ref[:n])


@pytest.mark.parametrize("index,sample", [(0, 4), (1, 10), (2, 8), (3, 6)])
def test_affine2_full_workloads(index, sample):
    w = WL.WORKLOADS[index]
    print(f"[parity] affine2 full workload {w.name} T={w.T}", flush=True)
    _EXPERTS_CACHE.clear()
    canon = WL.make_experts_affine2(w.seed, WL.N_EXPERTS)
    inp = WL.make_layer_inputs(w, experts=canon)
    ex = B.Experts.from_canonical(canon, WL.N_EXPERTS, WL.HIDDEN, WL.INTER, routed_affine2=True)
    r = LC.full_check(inp, ex, sample_tokens=sample, seed=index, routed_fmt="affine2", whole=4, y_all=True)
    assert r["ambiguous"] == 0
    print(f"[parity] affine2 {w.name}: rows max/mean rel {r['rows_err'][0]:.2e}/{r['rows_err'][1]:.2e}, "
          f"y max/mean rel {r['y_err'][0]:.2e}/{r['y_err'][1]:.2e}", flush=True)
    del r, ex
    torch.cuda.empty_cache()


# The four calls captured in a HIP graph (the library allocates nothing and
# issues no memsets) and replayed several times, with eager work and host
# synchronisation between replays and the outputs cleared to NaN before each:
# every replay must reproduce the eager layer bit for bit.  Decode and
# prefill kernel families.
@pytest.mark.parametrize("T", [37, 300])
def test_graph_replay_matches_eager(T):
    print(f"[parity] graph replay T={T}", flush=True)
    inp = _small_inputs(T, 512, 512, 16, 8100 + T)
    ex = _experts(inp)
    g = LC.run_gpu_layer(inp, ex)
    layer = g["layer"]
    y_ref = layer.y.clone()
    rows_ref = layer.out_rows.clone()
    n = int(g["offsets"][-1])
    xd = LC.dev(inp.x)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(xd)
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        layer.y.view(torch.uint8).fill_(0xFF)
        layer.out_rows.view(torch.uint8).fill_(0xFF)
        scratch.mul_(1.0001)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.y, y_ref), f"replay {rep}: y differs from the eager layer"
        assert torch.equal(layer.out_rows[:n], rows_ref[:n]), f"replay {rep}: expert rows differ"
