"""Host-side tests of the C ABI: the library loads and exports every declared
symbol, the repack is a bit-exact permutation that matches the documented
device layout, and every argument check returns its status without touching
a GPU (each refused call returns before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

from mxfp4_routed_expert_moe_amd import binding as B
from mxfp4_routed_expert_moe_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, EINVAL, EALIGN, ELAYOUT, ESHAPE, EWORKSPACE = 0, 1, 2, 3, 4, 5


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = _declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.EXPORTED)
    assert L.moe_abi_version() == B.MOE_ABI_VERSION


def test_status_strings():
    L = B.lib()
    for code, name in B.STATUS.items():
        assert L.moe_status_str(code).decode().startswith(name)
    assert L.moe_status_str(99) == b"unknown moe status"


def test_expert_bytes():
    assert B.expert_bytes(4096, 2048) == 13_369_344 == WL.expert_bytes(4096, 2048)
    assert B.expert_bytes(512, 512) == WL.expert_bytes(512, 512)
    assert B.expert_bytes(4096, 1000) == 0 and B.expert_bytes(0, 512) == 0 and B.expert_bytes(-512, 512) == 0


def _spec_tiled_offset(plane_nib_bytes, N, K, n, k, scale):
    """Device-layout offset (within a projection) of canonical nibble byte holding
    column k of row n, or of the scale of (n, k // 32), as the header states it."""
    if not scale:
        tile = (n // 16) * (K // 128) + k // 128
        lane = 16 * ((k % 128) // 32) + (n % 16)
        return tile * 1024 + lane * 16 + ((k % 32) // 2)
    grp = k // 32
    block = (n // 16) * (K // 512) + (k // 512)
    i = (grp % 16) // 4
    lane = (n % 16) + 16 * (grp % 4)
    return plane_nib_bytes + block * 256 + 4 * lane + i


@pytest.mark.parametrize("shape", [(512, 512), (1024, 512), (4096, 2048)])
def test_pack_matches_documented_layout_and_round_trips(shape):
    H, I = shape
    n_total = 2 if H < 4096 else 1
    blob = WL.make_experts(7, n_total, H, I, scale_lo=0, scale_hi=255)
    packed = B.pack_mxfp4(blob, n_total, H, I)
    assert packed.shape == blob.shape and not np.array_equal(packed, blob)
    assert np.array_equal(np.sort(packed), np.sort(blob))            # a permutation of the bytes
    assert np.array_equal(B.unpack_mxfp4(packed, n_total, H, I), blob)  # exact inverse
    off = WL.expert_plane_offsets(H, I)
    eb = WL.expert_bytes(H, I)
    g = np.random.default_rng(0)
    for xid in range(n_total):
        for proj, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            base = xid * eb + off[proj + "_nib"]
            for _ in range(200):
                n, k = int(g.integers(N)), int(g.integers(K))
                c_nib = base + n * (K // 2) + k // 2
                assert packed[base + _spec_tiled_offset(N * K // 2, N, K, n, k, False)] == blob[c_nib]
                c_sc = base + N * K // 2 + n * (K // 32) + k // 32
                assert packed[base + _spec_tiled_offset(N * K // 2, N, K, n, k, True)] == blob[c_sc]


def _spec_tiled8_offset(N, K, n, k, scale):
    """Where the device layout puts canonical MXFP8 code (n, k) (or its scale),
    from the description in include/moe.h, as an offset within the projection."""
    if scale:
        return N * K + _spec_tiled_offset(N * K // 2, N, K, n, k, True) - N * K // 2
    tile = (n // 16) * (K // 128) + k // 128
    g, half, r = (k % 128) // 32, (k % 32) // 16, n % 16
    return tile * 2048 + half * 1024 + (16 * g + r) * 16 + k % 16


@pytest.mark.parametrize("shape", [(512, 512), (1024, 512), (512, 1536)])
def test_pack_mxfp8_matches_documented_layout_and_round_trips(shape):
    H, I = shape
    blob = WL.make_shared_mxfp8(9, H, I, scale_lo=0, scale_hi=255)
    assert blob.nbytes == B.lib().moe_expert_bytes_mxfp8(H, I) == 3 * H * I * 33 // 32
    packed = B.pack_mxfp8(blob, H, I)
    assert not np.array_equal(packed, blob) and np.array_equal(np.sort(packed), np.sort(blob))
    assert np.array_equal(B.unpack_mxfp8(packed, H, I), blob)
    g = np.random.default_rng(1)
    base = 0
    for N, K in ((I, H), (I, H), (H, I)):
        for _ in range(300):
            n, k = int(g.integers(N)), int(g.integers(K))
            assert packed[base + _spec_tiled8_offset(N, K, n, k, False)] == blob[base + n * K + k]
            assert packed[base + _spec_tiled8_offset(N, K, n, k, True)] == blob[base + N * K + n * (K // 32) + k // 32]
        base += N * K + N * K // 32
    L = B.lib()
    n = blob.nbytes
    out = np.empty_like(blob)
    assert L.moe_pack_mxfp8(blob.ctypes.data, n - 1, H, I, out.ctypes.data, n) == EINVAL
    assert L.moe_pack_mxfp8(blob.ctypes.data, n, H, I + 1, out.ctypes.data, n) == ESHAPE
    assert L.moe_pack_mxfp8(blob.ctypes.data, n, H, I, blob.ctypes.data + 16, n) == EINVAL  # overlap
    assert L.moe_expert_bytes_mxfp8(4096, 2048) == 25_952_256 and L.moe_expert_bytes_mxfp8(4000, 2048) == 0


def _spec_affine2_code(packed, base, N, K, n, k):
    """Canonical 2-bit code (n, k) read from the device layout as include/moe.h
    describes it (512-byte tiles; lane 16g + r; word s // 2; the code of (s, i)
    at bit 4 i + 2 (s % 2))."""
    tile = (n // 16) * (K // 128) + k // 128
    kk = k % 128
    s_, g, i = kk // 32, (kk % 32) // 8, kk % 8
    word = base + tile * 512 + (16 * g + n % 16) * 8 + 4 * (s_ // 2)
    w = int.from_bytes(bytes(packed[word:word + 4]), "little")
    return (w >> (4 * i + 2 * (s_ % 2))) & 3


@pytest.mark.parametrize("shape", [(512, 512), (1024, 512), (512, 2048)])
def test_pack_affine2_matches_documented_layout_and_round_trips(shape):
    H, I = shape
    E = 2
    canon = WL.make_experts_affine2(11, E, H, I)[:E * H * I]
    assert B.lib().moe_expert_bytes_affine2(H, I) == H * I == WL.affine2_expert_bytes(H, I)
    packed = B.pack_affine2(canon, E, H, I)
    assert not np.array_equal(packed, canon)
    assert np.array_equal(B.unpack_affine2(packed, E, H, I), canon)
    g = np.random.default_rng(2)
    for x in range(E):
        base = x * H * I
        for (N, K), G in zip(((I, H), (I, H), (H, I)), (64, 64, 32)):
            for _ in range(200):
                n, k = int(g.integers(N)), int(g.integers(K))
                want = (int(canon[base + n * (K // 4) + k // 4]) >> (2 * (k % 4))) & 3
                assert _spec_affine2_code(packed, base, N, K, n, k) == want
                # (scale, bias) of (n, k): 16 * (128 / G) * 4-byte blocks, entry (n % 16) * (128 / G) + (k % 128) / G
                sb = base + N * K // 4
                blk = (n // 16) * (K // 128) + k // 128
                at = sb + blk * 16 * (128 // G) * 4 + ((n % 16) * (128 // G) + (k % 128) // G) * 4
                ng = N * K // G
                ci = n * (K // G) + k // G
                assert bytes(packed[at:at + 2]) == bytes(canon[sb + 2 * ci: sb + 2 * ci + 2])              # scale
                assert bytes(packed[at + 2:at + 4]) == bytes(canon[sb + 2 * ng + 2 * ci: sb + 2 * ng + 2 * ci + 2])
            base += N * K // 4 + 4 * (N * K // G)
    L = B.lib()
    n = canon.nbytes
    out = np.empty_like(canon)
    assert L.moe_pack_affine2(canon.ctypes.data, n - 1, E, H, I, out.ctypes.data, n) == EINVAL
    assert L.moe_pack_affine2(canon.ctypes.data, n, E, H, I + 1, out.ctypes.data, n) == ESHAPE
    assert L.moe_pack_affine2(canon.ctypes.data, n, 0, H, I, out.ctypes.data, n) == EINVAL
    assert L.moe_pack_affine2(canon.ctypes.data, n, E, H, I, canon.ctypes.data + 16, n) == EINVAL  # overlap
    assert L.moe_expert_bytes_affine2(4096, 2048) == 8_388_608 and L.moe_expert_bytes_affine2(4000, 2048) == 0
    assert L.moe_expert_bytes_affine2(B.MOE_MAX_DIM + 512, 512) == 0 and L.moe_expert_bytes(512, B.MOE_MAX_DIM + 512) == 0


def test_pack_rejects_bad_arguments():
    L = B.lib()
    a = np.zeros(B.expert_bytes(512, 512) * 2, dtype=np.uint8)
    b = np.zeros_like(a)
    n = a.nbytes
    assert L.moe_pack_mxfp4(None, n, 2, 512, 512, b.ctypes.data, n) == EINVAL
    assert L.moe_pack_mxfp4(a.ctypes.data, n, 0, 512, 512, b.ctypes.data, n) == EINVAL
    assert L.moe_pack_mxfp4(a.ctypes.data, n, 2, 500, 512, b.ctypes.data, n) == ESHAPE
    assert L.moe_pack_mxfp4(a.ctypes.data, n - 1, 2, 512, 512, b.ctypes.data, n) == EINVAL
    assert L.moe_pack_mxfp4(a.ctypes.data, n, 2, 512, 512, b.ctypes.data, n - 1) == EINVAL
    assert L.moe_pack_mxfp4(a.ctypes.data, n, 2, 512, 512, a.ctypes.data + 16, n) == EINVAL  # overlap
    assert L.moe_unpack_mxfp4(a.ctypes.data, n, 2, 512, 512, b.ctypes.data, n) == OK


# ---------------------------------------------------------------- argument checks (no GPU work)
FAKE = 0x7F0000000000          # never dereferenced: every call below is refused first
FAKE_MIS = FAKE + 8            # misaligned for 16/256-byte requirements


def _desc(**kw):
    d = B.moe_experts()
    assert B.lib().moe_experts_init(ctypes.byref(d), ctypes.c_void_p(FAKE), 256, 4096, 2048) == OK
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_experts_init_checks():
    L = B.lib()
    d = B.moe_experts()
    assert L.moe_experts_init(None, ctypes.c_void_p(FAKE), 256, 4096, 2048) == EINVAL
    assert L.moe_experts_init(ctypes.byref(d), None, 256, 4096, 2048) == EINVAL
    assert L.moe_experts_init(ctypes.byref(d), ctypes.c_void_p(FAKE), 0, 4096, 2048) == ESHAPE
    assert L.moe_experts_init(ctypes.byref(d), ctypes.c_void_p(FAKE), 256, 4000, 2048) == ESHAPE
    d = _desc()
    assert (d.abi_version, d.layout, d.n_experts, d.hidden, d.inter, d.expert_bytes) == (
        1, B.MOE_LAYOUT_GFX950_TILED_V1, 256, 4096, 2048, 13_369_344)


def _route(T=4, H=4096, x=FAKE, w=FAKE, bias=None, tok=None, table=None, V=0, E=256, k=6, scale=1.5,
           ids=FAKE, wt=FAKE, ws=FAKE, ws_bytes=1 << 40):
    v = lambda p: None if p is None else ctypes.c_void_p(p)  # noqa: E731
    return B.lib().moe_route(v(x), T, H, v(w), v(bias), v(tok), v(table), V, E, k, scale, v(ids), v(wt), v(ws),
                             ws_bytes, None)


def test_route_checks():
    assert _route(T=0) == OK                      # no-op
    assert _route(T=-1) == EINVAL
    assert _route(T=B.MOE_MAX_TOKENS + 1) == ESHAPE and B.lib().moe_route_workspace_size(B.MOE_MAX_TOKENS + 1,
                                                                                        4096, 256) == 0
    assert _route(k=0) == ESHAPE and _route(k=9) == ESHAPE
    assert _route(E=5) == ESHAPE and _route(E=257) == ESHAPE
    assert _route(scale=float("nan")) == EINVAL
    assert _route(ids=None) == EINVAL and _route(wt=None) == EINVAL
    assert _route(x=None) == EINVAL and _route(w=None) == EINVAL
    assert _route(H=4000) == ESHAPE
    assert _route(x=FAKE_MIS) == EALIGN
    assert _route(ws=None) == EINVAL and _route(ws=FAKE_MIS) == EALIGN
    need = B.lib().moe_route_workspace_size(4, 4096, 256)
    assert need > 0 and _route(ws_bytes=need - 1) == EWORKSPACE
    assert _route(table=FAKE, tok=None, V=10) == EINVAL
    assert _route(table=FAKE, tok=FAKE, V=0) == EINVAL


def _dispatch(T=64, E=256, k=6, ids=FAKE, off=FAKE, rt=FAKE, sr=FAKE, ws=FAKE, ws_bytes=1 << 40):
    v = lambda p: None if p is None else ctypes.c_void_p(p)  # noqa: E731
    return B.lib().moe_dispatch(v(ids), T, E, k, v(off), v(rt), v(sr), v(ws), ws_bytes, None)


def test_dispatch_checks():
    assert _dispatch(T=0) == OK
    assert _dispatch(T=-3) == EINVAL
    assert _dispatch(T=B.MOE_MAX_TOKENS + 1) == ESHAPE
    assert _dispatch(k=0) == ESHAPE and _dispatch(E=0) == ESHAPE and _dispatch(E=1024) == ESHAPE
    for name in ("ids", "off", "rt", "sr", "ws"):
        assert _dispatch(**{name: None}) == EINVAL
    assert _dispatch(ws=FAKE_MIS) == EALIGN
    need = B.lib().moe_dispatch_workspace_size(64, 256, 6)
    assert need > 0 and _dispatch(ws_bytes=need - 1) == EWORKSPACE


def _dispatch_noalloc(T=64, E=256, k=6, ids=FAKE, off=FAKE, rt=FAKE, sr=FAKE):
    v = lambda p: None if p is None else ctypes.c_void_p(p)  # noqa: E731
    return B.lib().moe_dispatch_noalloc(v(ids), T, E, k, v(off), v(rt), v(sr), None)


def test_dispatch_noalloc_checks():
    # refused calls return before any HIP call: no GPU needed
    assert _dispatch_noalloc(T=0) == OK
    assert _dispatch_noalloc(T=-3) == EINVAL
    assert _dispatch_noalloc(T=B.MOE_MAX_TOKENS + 1) == ESHAPE
    assert _dispatch_noalloc(k=9) == ESHAPE and _dispatch_noalloc(E=0) == ESHAPE
    for name in ("ids", "off", "rt", "sr"):
        assert _dispatch_noalloc(**{name: None}) == EINVAL
    # the static scratch holds what moe_dispatch's workspace would: calls
    # needing more are refused with MOE_EWORKSPACE
    cap = B.MOE_DISPATCH_NOALLOC_SCRATCH_BYTES
    L = B.lib()
    T_ok = max(T for T in range(140000, 160000, 64) if L.moe_dispatch_workspace_size(T, 256, 6) <= cap)
    assert T_ok > 140000
    assert _dispatch_noalloc(T=T_ok + 64) == EWORKSPACE
    assert _dispatch_noalloc(T=100000, E=1023, k=8) == EWORKSPACE


def _ffn(T=64, d=None, k=6, x=FAKE, off=FAKE, rt=FAKE, L=10.0, out=FAKE, ws=FAKE, ws_bytes=1 << 40):
    v = lambda p: None if p is None else ctypes.c_void_p(p)  # noqa: E731
    d = _desc() if d is None else d
    return B.lib().moe_expert_ffn(v(x), T, ctypes.byref(d), k, v(off), v(rt), L, v(out), v(ws), ws_bytes, None)


def test_ffn_checks():
    assert _ffn(T=0) == OK
    assert _ffn(T=-1) == EINVAL
    assert _ffn(d=_desc(layout=B.MOE_LAYOUT_CANONICAL_MXFP4)) == ELAYOUT   # wrong layout tag: fail loudly
    assert _ffn(d=_desc(layout=0x12345678)) == ELAYOUT
    assert _ffn(d=_desc(abi_version=2)) == ELAYOUT
    assert _ffn(d=_desc(expert_bytes=13_369_344 + 32)) == ESHAPE
    assert _ffn(d=_desc(hidden=4000)) == ESHAPE
    assert _ffn(d=_desc(n_experts=0)) == ESHAPE
    assert _ffn(d=_desc(flags=8)) == EINVAL and _ffn(d=_desc(flags=-1)) == EINVAL   # unknown flag bits
    assert _ffn(T=B.MOE_MAX_TOKENS + 1) == ESHAPE
    assert B.lib().moe_ffn_workspace_size(B.MOE_MAX_TOKENS + 1, ctypes.byref(_desc()), 6) == 0
    assert _ffn(d=_desc(flags=B.MOE_FFN_SPLIT_FP8 | B.MOE_SHARED_MXFP8)) == EINVAL  # not combinable
    assert _ffn(d=_desc(flags=B.MOE_SHARED_MXFP8), T=0) == OK
    # 2-bit affine routed experts: expert_bytes = H * I, decode-family K sizes only, no split option
    a2 = dict(flags=B.MOE_ROUTED_AFFINE2, expert_bytes=4096 * 2048)
    assert _ffn(d=_desc(**a2), T=0) == OK
    assert _ffn(d=_desc(flags=B.MOE_ROUTED_AFFINE2)) == ESHAPE                          # MXFP4 expert_bytes
    assert _ffn(d=_desc(**dict(a2, flags=B.MOE_ROUTED_AFFINE2 | B.MOE_SHARED_MXFP8)), T=0) == OK
    assert _ffn(d=_desc(**dict(a2, flags=B.MOE_ROUTED_AFFINE2 | B.MOE_FFN_SPLIT_FP8))) == EINVAL
    assert _ffn(d=_desc(flags=B.MOE_ROUTED_AFFINE2, hidden=1536, expert_bytes=1536 * 2048)) == ESHAPE
    d_ok = _desc(flags=B.MOE_ROUTED_AFFINE2, hidden=1536, expert_bytes=1536 * 2048)
    d_ok.flags = 0
    d_ok.expert_bytes = B.lib().moe_expert_bytes(1536, 2048)
    assert _ffn(d=d_ok, T=0) == OK                      # the same shape is fine for MXFP4 (prefill family)
    # the affine codec needs the same workspace as MXFP4 routed experts (work list and bf16 h)
    for T in (64, 4096):
        wa2 = B.lib().moe_ffn_workspace_size(T, ctypes.byref(_desc(**a2)), 6)
        assert wa2 == B.lib().moe_ffn_workspace_size(T, ctypes.byref(_desc()), 6) >= 7 * T * 2048 * 2
    assert _ffn(d=_desc(base=FAKE + 128)) == EALIGN
    assert _ffn(d=_desc(base=None)) == EINVAL
    assert _ffn(k=0) == ESHAPE and _ffn(k=9) == ESHAPE
    assert _ffn(L=0.0) == EINVAL and _ffn(L=float("nan")) == EINVAL
    for name in ("x", "off", "rt", "out", "ws"):
        assert _ffn(**{name: None}) == EINVAL
    assert _ffn(x=FAKE_MIS) == EALIGN and _ffn(out=FAKE_MIS) == EALIGN and _ffn(ws=FAKE + 64) == EALIGN
    need = B.lib().moe_ffn_workspace_size(64, ctypes.byref(_desc()), 6)
    assert need > 64 * 7 * 2048 * 2 and _ffn(ws_bytes=need - 1) == EWORKSPACE
    # MOE_FFN_SPLIT_FP8 changes only the prefill family's workspace: x and h
    # as two byte planes plus one scale byte per 32 (no bf16 h)
    split = _desc(flags=B.MOE_FFN_SPLIT_FP8)
    assert B.lib().moe_ffn_workspace_size(64, ctypes.byref(split), 6) == need
    T = 4096
    plain = B.lib().moe_ffn_workspace_size(T, ctypes.byref(_desc()), 6)
    two = B.lib().moe_ffn_workspace_size(T, ctypes.byref(split), 6)
    planes = lambda rows, K: 2 * rows * K + rows * K // 32  # noqa: E731
    assert two - plain == planes(T, 4096) + planes(7 * T, 2048) - 7 * T * 2048 * 2
    assert B.lib().moe_ffn_workspace_size(64, ctypes.byref(_desc(layout=1)), 6) == 0


def test_combine_checks():
    L = B.lib()
    v = ctypes.c_void_p
    f = lambda T=4, H=4096, k=6, o=FAKE, s=FAKE, w=FAKE, y=FAKE: L.moe_combine(  # noqa: E731
        None if o is None else v(o), None if s is None else v(s), None if w is None else v(w), T, H, k,
        None if y is None else v(y), None)
    assert f(T=0) == OK and f(T=-1) == EINVAL
    assert f(k=0) == ESHAPE and f(H=4095) == ESHAPE and f(T=B.MOE_MAX_TOKENS + 1) == ESHAPE
    assert f(o=None) == EINVAL and f(s=None) == EINVAL and f(w=None) == EINVAL and f(y=None) == EINVAL
    assert f(o=FAKE_MIS) == EALIGN and f(y=FAKE_MIS) == EALIGN


def test_binding_has_no_cpu_fallback(tmp_path, monkeypatch):
    # the product path refuses to run without the HIP library
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
