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
    """Host copy of a device tensor; bf16 tensors (the expert rows) come back
    as their exact float64 values."""
    import torch
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def poison(layer) -> None:
    """Fill every output and workspace of a MoeLayer with 0xFF bytes (float32
    and bf16 NaN, int32 -1), so that a row or token the kernels fail to write
    shows up as non-finite instead of as a stale value left by an earlier run.
    Every kernel writes what it later reads, and rows past an item re-read the
    item's last row, so no poisoned value is ever used as an index."""
    import torch
    for t in (layer.ids, layer.weights, layer.offsets, layer.row_token, layer.slot_row, layer.out_rows, layer.y,
              layer.ws_route, layer.ws_disp, layer.ws_ffn):
        t.view(-1).view(torch.uint8).fill_(0xFF)


def assert_all_written(layer, n_rows: int) -> None:
    """Every dispatched row of out_rows and every element of y is finite
    (checked on the device in slices, so even the largest batch needs no
    host copy)."""
    import torch
    step = 1 << 16
    for r0 in range(0, n_rows, step):
        blk = layer.out_rows[r0:min(n_rows, r0 + step)]
        assert bool(torch.isfinite(blk).all()), f"out_rows {r0}..{r0 + blk.shape[0]}: a row left unwritten (NaN)"
    yb = layer.y.view(torch.bfloat16)
    for t0 in range(0, yb.shape[0], step):
        assert bool(torch.isfinite(yb[t0:t0 + step]).all()), f"y tokens {t0}..: left unwritten (NaN)"


def run_gpu_layer(inp: WL.LayerInputs, experts: B.Experts, T: int | None = None, x=None, poisoned: bool = True):
    """All four calls through the C ABI; returns host copies of every output.
    With poisoned (the default) every output and workspace starts as NaN
    bytes and the run must leave every dispatched row and every output
    finite."""
    import torch
    T = inp.x.shape[0] if T is None else T
    layer = B.MoeLayer(experts, T, inp.top_k, WL.ROUTE_SCALE, WL.CLAMP_LIMIT,
                       w_router=None if inp.router is None else dev(inp.router),
                       sel_bias=None if inp.bias is None else dev(inp.bias),
                       hash_table=None if inp.table is None else dev(inp.table))
    if poisoned:
        poison(layer)
    xd = dev(inp.x) if x is None else x
    tok = None if inp.tok is None else dev(inp.tok)
    layer.forward(xd, tok)
    torch.cuda.synchronize()
    offsets = host(layer.offsets)
    if poisoned:
        assert_all_written(layer, int(offsets[-1]))
    return dict(ids=host(layer.ids), weights=host(layer.weights), offsets=offsets,
                row_token=host(layer.row_token), slot_row=host(layer.slot_row), out_rows=layer.out_rows,
                y=host(layer.y).view(np.uint16), layer=layer)


def oracle_routing(inp: WL.LayerInputs, toks=None):
    """Oracle ids, weights and selection gaps of every token, or of the tokens
    toks (routing is per token, so a subset is computed on its own)."""
    x = inp.x if toks is None else inp.x[toks]
    if inp.table is not None:
        tok = inp.tok if toks is None else inp.tok[toks]
        ids, w = O.route_hash(tok, inp.table, inp.top_k, WL.ROUTE_SCALE)
        gap = np.full(len(ids), np.inf)
    else:
        ids, w, _ = O.route_learned(x, inp.router, inp.bias, inp.top_k, WL.ROUTE_SCALE)
        gap = O.boundary_gap(x, inp.router, inp.bias, inp.top_k)
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


def check_routing(g, ids_ref, w_ref, gap, toks=None):
    """Bit-exact ids (tokens on a near tie, if any, are reported and skipped);
    ids_ref, w_ref and gap cover every token, or the tokens toks."""
    ids = g["ids"] if toks is None else g["ids"][toks]
    wts = g["weights"] if toks is None else g["weights"][toks]
    clear = gap >= AMBIGUOUS_GAP
    assert clear.mean() > 0.99
    assert np.array_equal(ids[clear], ids_ref[clear])
    wr = w_ref[clear]
    assert np.max(np.abs(wts[clear] - wr) / np.abs(wr)) <= W_REL
    return int((~clear).sum())


def check_dispatch(g, ids_gpu, E):
    off, rt, sr = O.dispatch(ids_gpu, E)
    assert np.array_equal(g["offsets"], off)
    n = int(off[-1])
    assert np.array_equal(g["row_token"][:n], rt)
    assert np.array_equal(g["slot_row"], sr)
    return off, rt, sr


def pick_whole_experts(off: np.ndarray, n_experts: int, n_ragged: int, seed: int = 0, big: bool = True) -> list:
    """Groups whose rows are all compared with the oracle: the hottest routed
    expert and the shared expert (unless big is False), the smallest non-empty
    routed expert and n_ragged random routed experts whose row count is not a
    multiple of 64 (a ragged last prefill item)."""
    cnt = np.diff(off[: n_experts + 1])
    live = np.nonzero(cnt > 0)[0]
    pick = ([int(np.argmax(cnt)), n_experts] if big else []) + [int(live[np.argmin(cnt[live])])]
    ragged = [int(e) for e in live if cnt[e] % 64 != 0 and int(e) not in pick]
    rng = np.random.default_rng([seed, 2])
    pick += [int(e) for e in rng.choice(ragged, min(n_ragged, len(ragged)), replace=False)]
    return list(dict.fromkeys(pick))


def check_whole_experts(inp: WL.LayerInputs, g, off, rt, groups, shared_fmt="mxfp4", routed_fmt="mxfp4",
                        chunk: int = 4096):
    """Every row of each group in groups against the oracle's expert, in row
    slices of `chunk`.  Returns the worst (max, mean) relative error."""
    worst = (0.0, 0.0)
    for e in groups:
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        fmt = shared_fmt if e == inp.n_experts else routed_fmt
        mats = O.decode_expert(inp.experts, e, inp.hidden, inp.inter, fmt, routed_fmt)
        for a in range(r0, r1, chunk):
            b = min(r1, a + chunk)
            want = O.expert_forward(O.bf16_bits_to_f64(inp.x[rt[a:b]]), mats, WL.CLAMP_LIMIT)
            got = host(g["out_rows"][a:b])
            err = assert_output_close(got, want, f"expert {e} rows {a}..{b} of {r0}..{r1}")
            worst = (max(worst[0], err[0]), max(worst[1], err[1]))
    return worst


def check_combine_all(g, sr, w_ref, toks=None, chunk: int = 2048):
    """y of every token (or of the tokens toks) against the oracle's combine of
    the GPU's own expert rows with the oracle's routing weights (w_ref: one row
    per token of toks).  Returns the worst (max, mean) relative error."""
    import torch
    toks = np.arange(sr.shape[0]) if toks is None else np.asarray(toks)
    worst = (0.0, 0.0)
    for a in range(0, len(toks), chunk):
        tk = toks[a:a + chunk]
        srs = sr[tk].astype(np.int64)
        used = np.unique(srs[srs >= 0])
        rows = host(g["out_rows"][torch.from_numpy(used).to(g["out_rows"].device)]).astype(np.float64)
        src = np.where(srs >= 0, np.searchsorted(used, srs), -1)
        y_ref = O.combine(rows, src, w_ref[a:a + chunk])
        err = assert_output_close(O.bf16_bits_to_f64(g["y"][tk]), y_ref, f"combine of tokens {tk[0]}..{tk[-1]}")
        worst = (max(worst[0], err[0]), max(worst[1], err[1]))
    return worst


def full_check(inp: WL.LayerInputs, experts: B.Experts, sample_tokens=None, seed=0, shared_fmt="mxfp4",
               routed_fmt="mxfp4", route_sample=None, whole=None, whole_big=True, y_all=False):
    """Whole-layer parity: routing, dispatch, expert rows and y.  With
    sample_tokens, the expert rows and outputs are checked on that many
    randomly chosen tokens (the oracle computes each one on its own).  With
    route_sample, the routing is checked on that many random tokens plus the
    first and the last (dispatch is still checked on every pair, from the
    GPU's ids).  shared_fmt, routed_fmt: the weight formats of the shared and
    the routed experts in inp.experts.  With whole = n, every row of the
    groups pick_whole_experts(offsets, E, n, seed, whole_big) chooses is
    compared too; with
    y_all, y of every routing-checked token is compared with the oracle's
    combine of the GPU's rows.  Every run starts from NaN-filled outputs and
    workspaces and must leave every dispatched row and every output finite."""
    g = run_gpu_layer(inp, experts)
    T = inp.x.shape[0]
    if route_sample is None or route_sample >= T:
        rtoks = np.arange(T)
    else:
        pick = np.random.default_rng([seed, 1]).choice(T, route_sample, replace=False)
        rtoks = np.unique(np.concatenate([pick, [0, T - 1]]))
    ids_ref, w_ref, gap = oracle_routing(inp, None if len(rtoks) == T else rtoks)
    n_amb = check_routing(g, ids_ref, w_ref, gap, None if len(rtoks) == T else rtoks)
    off, rt, sr = check_dispatch(g, g["ids"], inp.n_experts)
    # rows and y on a sample of the routing-checked tokens (positions in rtoks)
    if sample_tokens is None or sample_tokens >= len(rtoks):
        pos = np.arange(len(rtoks))
    else:
        pos = np.sort(np.random.default_rng(seed).choice(len(rtoks), sample_tokens, replace=False))
    pos = pos[gap[pos] >= AMBIGUOUS_GAP]      # a token on a near tie has two correct answers
    toks = rtoks[pos]
    rows = sr[toks].reshape(-1)
    rows = rows[rows >= 0]
    # oracle expert rows for the sampled rows only, expert-major
    ref_rows = {}
    grp = np.searchsorted(off, rows, side="right") - 1
    for e in np.unique(grp):
        fmt = shared_fmt if int(e) == inp.n_experts else routed_fmt
        mats = O.decode_expert(inp.experts, int(e), inp.hidden, inp.inter, fmt, routed_fmt)
        rs = rows[grp == e]
        o = O.expert_forward(O.bf16_bits_to_f64(inp.x[rt[rs]]), mats, WL.CLAMP_LIMIT)
        for r, v in zip(rs, o):
            ref_rows[int(r)] = v
    kept = np.asarray(sorted(ref_rows), dtype=np.int64)
    got_rows = host(g["out_rows"][kept])
    want_rows = np.stack([ref_rows[int(r)] for r in kept])
    rows_err = assert_output_close(got_rows, want_rows, "expert rows")
    # y of the sampled tokens from the oracle's rows and the oracle's weights
    # (routing matched, so the GPU's ids index the same rows); the rows are
    # held compactly, slot_row renumbered to match (dropped slots stay -1)
    sr_s = sr[toks].astype(np.int64)
    sr_c = np.where(sr_s >= 0, np.searchsorted(kept, sr_s), -1)
    y_ref = O.combine(want_rows, sr_c, w_ref[pos])
    y_got = O.bf16_bits_to_f64(g["y"][toks])
    y_err = assert_output_close(y_got, y_ref, "layer output")
    out = dict(g=g, rows_err=rows_err, y_err=y_err, ambiguous=n_amb, tokens=toks)
    if whole is not None:
        groups = pick_whole_experts(off, inp.n_experts, whole, seed, whole_big)
        out["whole_groups"] = groups
        out["whole_err"] = check_whole_experts(inp, g, off, rt, groups, shared_fmt, routed_fmt)
    if y_all:
        clear = gap >= AMBIGUOUS_GAP
        out["combine_err"] = check_combine_all(g, sr, w_ref[clear], rtoks[clear])
    return out
