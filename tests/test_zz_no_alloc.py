"""moe_dispatch_noalloc (the dispatch whose scratch lives in the library's
static device array, for callers that cannot allocate) against moe_dispatch
with a caller workspace, through the C ABI: bit-identical offsets, row_token
and slot_row on consecutive calls that reuse the same static scratch, the
second and third on smaller inputs than the first."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mxfp4_routed_expert_moe_amd import binding as B  # noqa: E402

pytestmark = pytest.mark.gpu


def _ids(T, E, k, seed):
    g = np.random.default_rng(seed)
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    drop = g.random((T, k)) < 0.01            # a few dropped ids (-1 or out of range)
    ids[drop] = np.where(g.random(int(drop.sum())) < 0.5, -1, E + 3)
    return torch.from_numpy(ids).cuda()


def test_noalloc_dispatch_matches_workspace_dispatch():
    E, k = 256, 6
    # large path (three kernels, scratch used), then smaller ones reusing the
    # scratch: a smaller large-path call and a single-block call
    for i, T in enumerate((20000, 3001, 100)):
        print(f"[noalloc] dispatch T={T} E={E} k={k}", flush=True)
        ids = _ids(T, E, k, 40 + i)
        ref = B.dispatch(ids, E)
        got = B.dispatch_noalloc(ids, E)
        torch.cuda.synchronize()
        n = int(ref[0][-1].item())
        assert torch.equal(got[0], ref[0])
        assert torch.equal(got[1][:n], ref[1][:n])
        assert torch.equal(got[2], ref[2])


def test_noalloc_dispatch_refuses_beyond_its_scratch():
    ids = torch.zeros((160000, 6), dtype=torch.int32, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.dispatch_noalloc(ids, 256)
    assert e.value.status == 5   # MOE_EWORKSPACE, nothing enqueued
