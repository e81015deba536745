"""Seeded random layer shapes on the GPU against the CPU oracle, element by
element: H and I among the supported multiples of 512 (1536 has no decode
variant, so it always takes the prefill family), E not a multiple of 64,
top_k from 1 to 8, learned or hash routing, with and without the selection
bias, and each descriptor option; a second sweep holds the routed experts in
the 2-bit affine codec.  The cases are drawn once from a fixed
seed, so a failure names a reproducible shape."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import moe_oracle as O  # noqa: E402
from mxfp4_routed_expert_moe_amd import binding as B  # noqa: E402
from mxfp4_routed_expert_moe_amd import workloads as WL  # noqa: E402
from tests import layer_check as LC  # noqa: E402

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.choice([512, 1024, 1536]))
        I = int(rng.choice([512, 1024, 1536]))
        E = int(rng.choice([7, 16, 33, 64, 100]))
        k = int(rng.integers(1, min(8, E) + 1))
        T = int(rng.choice([1, 3, 9, 40, 130, 260]))
        routing = "hash" if rng.random() < 0.3 else "learned"
        bias = routing == "learned" and rng.random() < 0.4
        opt = str(rng.choice(["none", "split_fp8", "shared_mxfp8"]))
        out.append((i, T, H, I, E, k, routing, bias, opt))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "-".join(str(v) for v in c))
def test_random_layer_against_oracle(case):
    i, T, H, I, E, k, routing, bias, opt = case
    print(f"[parity] random case {case}", flush=True)
    seed = 7000 + i
    x = WL.make_x(seed, T, H)
    router = b = table = tok = None
    if routing == "learned":
        router = WL.make_router(seed, H, E)
        if bias:
            b = (np.random.default_rng(seed).standard_normal(E) * 0.5).astype(np.float32)
    else:
        table, tok = WL.make_hash(seed, T, E, k, vocab=500)
    shared8 = opt == "shared_mxfp8"
    experts = WL.make_experts_shared_mxfp8(seed, E, H, I) if shared8 else WL.make_experts(seed, E + 1, H, I)
    w = WL.Workload(91, "random", T, routing, None)
    inp = WL.LayerInputs(w, x, router, b, table, tok, experts, H, I, E, k)
    ex = B.Experts.from_canonical(experts, E, H, I, split_fp8=opt == "split_fp8", shared_mxfp8=shared8)
    fmt = "mxfp8" if shared8 else "mxfp4"
    r = LC.full_check(inp, ex, shared_fmt=fmt)
    ref = O.moe_layer(x, experts, n_experts=E, hidden=H, inter=I, top_k=k, route_scale=WL.ROUTE_SCALE,
                      limit=WL.CLAMP_LIMIT, w_router=router, bias=b, token_ids=tok, table=table, shared_fmt=fmt)
    g = r["g"]
    if r["ambiguous"] == 0:
        n = int(ref["offsets"][-1])
        assert np.array_equal(g["offsets"], ref["offsets"]) and np.array_equal(g["row_token"][:n], ref["row_token"])
        LC.assert_output_close(LC.host(g["out_rows"][:n]), ref["out_rows"], "all rows")
        LC.assert_output_close(O.bf16_bits_to_f64(g["y"]), ref["y"], "all outputs")


def _cases_affine2(n=12, seed=2025):
    """The 2-bit affine routed experts: H and I among the decode-family sizes,
    the shared expert MXFP4 or MXFP8."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.choice([512, 1024, 2048]))
        I = int(rng.choice([512, 1024, 2048]))
        E = int(rng.choice([7, 16, 33, 64, 100]))
        k = int(rng.integers(1, min(8, E) + 1))
        T = int(rng.choice([1, 3, 9, 40, 130, 260]))
        routing = "hash" if rng.random() < 0.3 else "learned"
        bias = routing == "learned" and rng.random() < 0.4
        shared = str(rng.choice(["mxfp4", "mxfp8"]))
        out.append((i, T, H, I, E, k, routing, bias, shared))
    return out


@pytest.mark.parametrize("case", _cases_affine2(), ids=lambda c: "-".join(str(v) for v in c))
def test_random_affine2_layer_against_oracle(case):
    i, T, H, I, E, k, routing, bias, shared = case
    print(f"[parity] random affine2 case {case}", flush=True)
    seed = 8000 + i
    x = WL.make_x(seed, T, H)
    router = b = table = tok = None
    if routing == "learned":
        router = WL.make_router(seed, H, E)
        if bias:
            b = (np.random.default_rng(seed).standard_normal(E) * 0.5).astype(np.float32)
    else:
        table, tok = WL.make_hash(seed, T, E, k, vocab=500)
    experts = WL.make_experts_affine2(seed, E, H, I, shared)
    w = WL.Workload(92, "random_affine2", T, routing, None)
    inp = WL.LayerInputs(w, x, router, b, table, tok, experts, H, I, E, k)
    ex = B.Experts.from_canonical(experts, E, H, I, shared_mxfp8=shared == "mxfp8", routed_affine2=True)
    r = LC.full_check(inp, ex, shared_fmt=shared, routed_fmt="affine2")
    ref = O.moe_layer(x, experts, n_experts=E, hidden=H, inter=I, top_k=k, route_scale=WL.ROUTE_SCALE,
                      limit=WL.CLAMP_LIMIT, w_router=router, bias=b, token_ids=tok, table=table, shared_fmt=shared,
                      routed_fmt="affine2")
    g = r["g"]
    if r["ambiguous"] == 0:
        n = int(ref["offsets"][-1])
        assert np.array_equal(g["offsets"], ref["offsets"]) and np.array_equal(g["row_token"][:n], ref["row_token"])
        LC.assert_output_close(LC.host(g["out_rows"][:n]), ref["out_rows"], "all rows")
        LC.assert_output_close(O.bf16_bits_to_f64(g["y"]), ref["y"], "all outputs")
