"""Shared helpers of the GPU parity tests and the smoke check: run the layer
through the C ABI, run the oracle on the same seeded inputs, and compare with
the parity bar (ids and dispatch bit-exact; routing weights within 1e-6
relative; outputs within max|d|/max|ref| <= 2e-2 and sum|d|/sum|ref| <= 5e-3).
"""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as O
from mxfp4_routed_expert_moe_amd import binding as B
from mxfp4_routed_expert_moe_amd import workloads as WL

MAX_REL = 2e-2
MEAN_REL = 5e-3
W_REL = 1e-6
AMBIGUOUS_GAP = 1e-9


def dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t) -> np.ndarray:
    return t.cpu().numpy()


def run_gpu_layer(inp: WL.LayerInputs, experts: B.Experts, T: int | None = None, x=None):
    """All four calls through the C ABI; returns host copies of every output."""
    import torch
    T = inp.x.shape[0] if T is None else T
    layer = B.MoeLayer(experts, T, inp.top_k, WL.ROUTE_SCALE, WL.CLAMP_LIMIT,
                       w_router=None if inp.router is None else dev(inp.router),
                       sel_bias=None if inp.bias is None else dev(inp.bias),
                       hash_table=None if inp.table is None else dev(inp.table))
    xd = dev(inp.x) if x is None else x
    tok = None if inp.tok is None else dev(inp.tok)
    layer.forward(xd, tok)
    torch.cuda.synchronize()
    return dict(ids=host(layer.ids), weights=host(layer.weights), offsets=host(layer.offsets),
                row_token=host(layer.row_token), slot_row=host(layer.slot_row), out_rows=layer.out_rows,
                y=host(layer.y).view(np.uint16), layer=layer)


def oracle_routing(inp: WL.LayerInputs):
    if inp.table is not None:
        ids, w = O.route_hash(inp.tok, inp.table, inp.top_k, WL.ROUTE_SCALE)
        gap = np.full(len(ids), np.inf)
    else:
        ids, w, _ = O.route_learned(inp.x, inp.router, inp.bias, inp.top_k, WL.ROUTE_SCALE)
        gap = O.boundary_gap(inp.x, inp.router, inp.bias, inp.top_k)
    return ids, w, gap


def rel_errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(np.asarray(got, dtype=np.float64) - ref)
    mx = float(d.max() / max(np.abs(ref).max(), 1e-300))
    mean = float(d.sum() / max(np.abs(ref).sum(), 1e-300))
    return mx, mean


def assert_output_close(got, ref, what=""):
    mx, mean = rel_errors(got, ref)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{what}: non-finite output"
    assert mx <= MAX_REL and mean <= MEAN_REL, f"{what}: max rel {mx:.3e}, mean rel {mean:.3e}"
    return mx, mean


def check_routing(g, ids_ref, w_ref, gap):
    """Bit-exact ids (tokens on a near tie, if any, are reported and skipped)."""
    clear = gap >= AMBIGUOUS_GAP
    assert clear.mean() > 0.99
    assert np.array_equal(g["ids"][clear], ids_ref[clear])
    wr = w_ref[clear]
    assert np.max(np.abs(g["weights"][clear] - wr) / np.abs(wr)) <= W_REL
    return int((~clear).sum())


def check_dispatch(g, ids_gpu, E):
    off, rt, sr = O.dispatch(ids_gpu, E)
    assert np.array_equal(g["offsets"], off)
    n = int(off[-1])
    assert np.array_equal(g["row_token"][:n], rt)
    assert np.array_equal(g["slot_row"], sr)
    return off, rt, sr


def full_check(inp: WL.LayerInputs, experts: B.Experts, sample_tokens=None, seed=0, shared_fmt="mxfp4",
               routed_fmt="mxfp4"):
    """Whole-layer parity: routing, dispatch, expert rows and y.  With
    sample_tokens, the expert rows and outputs are checked on that many
    randomly chosen tokens (the oracle computes each one on its own).
    shared_fmt, routed_fmt: the weight formats of the shared and the routed
    experts in inp.experts."""
    g = run_gpu_layer(inp, experts)
    ids_ref, w_ref, gap = oracle_routing(inp)
    n_amb = check_routing(g, ids_ref, w_ref, gap)
    off, rt, sr = check_dispatch(g, g["ids"], inp.n_experts)
    T = inp.x.shape[0]
    if sample_tokens is None or sample_tokens >= T:
        toks = np.arange(T)
    else:
        toks = np.sort(np.random.default_rng(seed).choice(T, sample_tokens, replace=False))
    toks = toks[gap[toks] >= AMBIGUOUS_GAP]      # a token on a near tie has two correct answers
    rows = sr[toks].reshape(-1)
    rows = rows[rows >= 0]
    # oracle expert rows for the sampled rows only, expert-major
    x = inp.x
    xf = O.bf16_bits_to_f64(x)
    ref_rows = {}
    grp = np.searchsorted(off, rows, side="right") - 1
    for e in np.unique(grp):
        fmt = shared_fmt if int(e) == inp.n_experts else routed_fmt
        mats = O.decode_expert(inp.experts, int(e), inp.hidden, inp.inter, fmt, routed_fmt)
        rs = rows[grp == e]
        o = O.expert_forward(xf[rt[rs]], mats, WL.CLAMP_LIMIT)
        for r, v in zip(rs, o):
            ref_rows[int(r)] = v
    got_rows = host(g["out_rows"][np.asarray(sorted(ref_rows), dtype=np.int64)])
    want_rows = np.stack([ref_rows[r] for r in sorted(ref_rows)])
    rows_err = assert_output_close(got_rows, want_rows, "expert rows")
    # y of the sampled tokens from the oracle's rows and the oracle's weights
    # (routing matched, so the GPU's ids index the same rows)
    out_s = np.zeros((int(off[-1]), inp.hidden))
    for r, v in ref_rows.items():
        out_s[r] = v
    w_use = w_ref.copy()
    y_ref = O.combine(out_s, sr[toks], w_use[toks])
    y_got = O.bf16_bits_to_f64(g["y"][toks])
    y_err = assert_output_close(y_got, y_ref, "layer output")
    return dict(g=g, rows_err=rows_err, y_err=y_err, ambiguous=n_amb, tokens=toks)
