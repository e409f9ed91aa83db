"""The C ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before any launch (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

from chunk_gated_delta_amd import carve

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "carve.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4
FAKE = 0x100000  # 16-byte aligned placeholder address; never dereferenced on a rejected call


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(carve_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return carve.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"carve_fwd", "carve_bwd", "carve_fwd_workspace_size", "carve_bwd_workspace_size",
            "carve_status_string", "carve_abi_version", "carve_fwd_ex", "carve_bwd_ex", "carve_fwd_save",
            "carve_bwd_saved", "carve_saved_size", "carve_bwd_saved_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.carve_abi_version() == 3
    for code in range(5):
        assert carve.status_string(code).startswith("CARVE_")


def shape(B=2, H=2, T=128, D=128, L=64, dtype=carve.CARVE_BF16, Dv=None):
    return carve.carve_shape(B, H, T, D, D if Dv is None else Dv, L, dtype)


def call_fwd(lib, s, q=FAKE, k=FAKE, v=FAKE, log_g=FAKE, b=None, w=FAKE, S0=None, content=None, o=FAKE,
             S_T=None, ws=FAKE, ws_bytes=1 << 40):
    return lib.carve_fwd(ctypes.byref(s), q, k, v, log_g, b, w, S0,
                         ctypes.byref(content) if content is not None else None, o, S_T, ws, ws_bytes, None)


def test_fwd_rejects_bad_shapes(lib):
    assert call_fwd(lib, shape(D=96)) == UNSUPPORTED
    assert call_fwd(lib, shape(D=128, Dv=96)) == UNSUPPORTED
    assert call_fwd(lib, shape(D=64, Dv=32)) == UNSUPPORTED
    assert call_fwd(lib, shape(B=-1)) == INVALID
    assert call_fwd(lib, shape(T=-5)) == INVALID
    assert call_fwd(lib, shape(L=0)) == INVALID
    assert call_fwd(lib, shape(dtype=7)) == INVALID
    assert call_fwd(lib, None if False else shape(), q=None) == INVALID
    assert call_fwd(lib, shape(), w=None) == INVALID
    assert call_fwd(lib, shape(), o=None) == INVALID
    assert call_fwd(lib, shape(), k=FAKE + 4) == INVALID          # misaligned


def test_fwd_workspace_checks(lib):
    s = shape()
    need = lib.carve_fwd_workspace_size(ctypes.byref(s), None)
    assert need > 0
    assert call_fwd(lib, s, ws_bytes=need - 1) == WORKSPACE
    assert call_fwd(lib, s, ws=None, ws_bytes=need) == WORKSPACE
    # the factor workspace scales with the token count
    s2 = shape(T=256)
    assert lib.carve_fwd_workspace_size(ctypes.byref(s2), None) > need
    # an empty problem needs no workspace and, with no outputs to fill, launches nothing
    s0 = shape(T=0)
    assert lib.carve_fwd_workspace_size(ctypes.byref(s0), None) == 0
    assert call_fwd(lib, s0, q=None, k=None, v=None, log_g=None, w=None, o=None, ws=None, ws_bytes=0) == OK
    sb = shape(B=0)
    assert call_fwd(lib, sb, q=None, k=None, v=None, log_g=None, w=None, o=None, ws=None, ws_bytes=0) == OK


def test_segmented_forward_workspace(lib):
    """Few heads and a long sequence: the forward workspace also holds the fp32 affine
    maps [C; Pi] and entering states of the state-pass segments, so per head it is
    larger than for a batch wide enough to run one sequential pass per head."""
    T = 64 * 100
    few, many = shape(B=1, H=2, T=T), shape(B=16, H=2, T=T)
    per_head_few = lib.carve_fwd_workspace_size(ctypes.byref(few), None) / 2
    per_head_many = lib.carve_fwd_workspace_size(ctypes.byref(many), None) / 32
    assert per_head_few > per_head_many + 3 * 128 * 128 * 4       # at least one segment's buffers
    # short sequences stay sequential (no segment buffers)
    short_few, short_many = shape(B=1, H=2, T=64 * 8), shape(B=16, H=2, T=64 * 8)
    assert abs(lib.carve_fwd_workspace_size(ctypes.byref(short_few), None) / 2 -
               lib.carve_fwd_workspace_size(ctypes.byref(short_many), None) / 32) < 4096


def test_fwd_content_checks(lib):
    c = carve.carve_content(FAKE, FAKE, FAKE, 16, None, None)
    assert call_fwd(lib, shape(), b=FAKE, content=c) == INVALID               # b together with content
    c_half = carve.carve_content(FAKE, FAKE, None, 16, None, None)
    assert call_fwd(lib, shape(), content=c_half) == INVALID                 # U1 without U2
    c_rank = carve.carve_content(FAKE, FAKE, FAKE, 0, None, None)
    assert call_fwd(lib, shape(), content=c_rank) == INVALID                 # rank 0
    c_nobx = carve.carve_content(None, None, None, 0, None, None)
    assert call_fwd(lib, shape(), content=c_nobx) == INVALID                 # b_x required
    c_rec = carve.carve_content(FAKE, FAKE, FAKE, 16, None, None, FAKE, None)
    assert call_fwd(lib, shape(), content=c_rec) == INVALID                  # z_rec without m_rec
    c_mis = carve.carve_content(FAKE, FAKE, FAKE, 16, None, None, FAKE, FAKE + 8)
    assert call_fwd(lib, shape(), content=c_mis) == INVALID                  # misaligned record
    assert call_fwd(lib, shape(L=16), content=c) == UNSUPPORTED               # period not whole tiles
    assert call_fwd(lib, shape(L=96), content=c) == UNSUPPORTED
    s = shape()
    assert lib.carve_fwd_workspace_size(ctypes.byref(s), ctypes.byref(c)) < \
        lib.carve_fwd_workspace_size(ctypes.byref(s), None)                  # one factor slot per head
    assert call_fwd(lib, s, content=c, ws_bytes=0) == WORKSPACE


def call_bwd(lib, s, b=None, db=None, dq=FAKE, dO=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.carve_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, b, FAKE, None, dO, None,
                         dq, FAKE, FAKE, FAKE, db, FAKE, None, ws, ws_bytes, None)


def test_bwd_checks(lib):
    s = shape()
    assert call_bwd(lib, s, b=FAKE, db=None) == INVALID        # db must be given iff b is
    assert call_bwd(lib, s, b=None, db=FAKE) == INVALID
    assert call_bwd(lib, s, dq=None) == INVALID
    assert call_bwd(lib, s, dO=None) == INVALID
    assert call_bwd(lib, shape(D=32)) == UNSUPPORTED
    need = lib.carve_bwd_workspace_size(ctypes.byref(s))
    assert need > lib.carve_fwd_workspace_size(ctypes.byref(s), None)
    assert call_bwd(lib, s, ws_bytes=need - 1) == WORKSPACE


def test_saved_pair_checks(lib):
    s = shape()
    need = lib.carve_saved_size(ctypes.byref(s))
    assert need > lib.carve_fwd_workspace_size(ctypes.byref(s), None)
    wsz = lib.carve_bwd_saved_workspace_size(ctypes.byref(s))
    assert 0 < wsz < lib.carve_bwd_workspace_size(ctypes.byref(s))
    # fwd_save: short saved buffer, misaligned input, missing output
    assert lib.carve_fwd_save(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE,
                              need - 1, None, None) == WORKSPACE
    assert lib.carve_fwd_save(ctypes.byref(s), FAKE, FAKE + 2, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE,
                              need, None, None) == INVALID
    assert lib.carve_fwd_save(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, None, FAKE,
                              need, None, None) == INVALID
    # bwd_saved: short saved buffer, short workspace, db without b
    args = lambda saved_b, ws_b, db: (ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, saved_b,
                                      FAKE, FAKE, FAKE, FAKE, db, FAKE, None, FAKE, ws_b, None, None)
    assert lib.carve_bwd_saved(*args(need - 1, wsz, None)) == WORKSPACE
    assert lib.carve_bwd_saved(*args(need, wsz - 1, None)) == WORKSPACE
    assert lib.carve_bwd_saved(*args(need, wsz, FAKE)) == INVALID


def call_decode(lib, s, q=FAKE, k=FAKE, v=FAKE, log_g=FAKE, b=None, w=FAKE, S=FAKE, content=None, o=FAKE):
    return lib.carve_decode_step(ctypes.byref(s), q, k, v, log_g, b, w, S,
                                 ctypes.byref(content) if content is not None else None, o, None)


def test_decode_rejects_bad_arguments(lib):
    assert call_decode(lib, shape(T=2)) == INVALID                 # one token per call
    assert call_decode(lib, shape(T=1, D=96)) == UNSUPPORTED
    assert call_decode(lib, shape(T=1), S=None) == INVALID
    assert call_decode(lib, shape(T=1), S=FAKE + 8) == INVALID     # state must be 16-byte aligned
    assert call_decode(lib, shape(T=1), o=None) == INVALID
    assert call_decode(lib, shape(T=1, B=0), q=None, k=None, v=None, log_g=None, w=None, S=None, o=None) == OK
    c = carve.carve_decode_content(FAKE, None, None, 0, FAKE, FAKE + 256, FAKE + 512, 0)
    assert call_decode(lib, shape(T=1, L=4), content=c, b=FAKE) == INVALID    # b comes from the content gate
    bad_pos = carve.carve_decode_content(FAKE, None, None, 0, FAKE, FAKE + 256, FAKE + 512, 4)
    assert call_decode(lib, shape(T=1, L=4), content=bad_pos) == INVALID
    alias = carve.carve_decode_content(FAKE, None, None, 0, FAKE, FAKE, FAKE + 512, 0)
    assert call_decode(lib, shape(T=1, L=4), content=alias) == INVALID        # m_out aliases m_in
    half = carve.carve_decode_content(FAKE, FAKE, None, 16, None, FAKE + 256, FAKE + 512, 0)
    assert call_decode(lib, shape(T=1, L=4), content=half) == INVALID         # U1 without U2
    rank = carve.carve_decode_content(FAKE, FAKE, FAKE, 65, None, FAKE + 256, FAKE + 512, 0)
    assert call_decode(lib, shape(T=1, L=4), content=rank) == INVALID
    no_sum = carve.carve_decode_content(FAKE, None, None, 0, None, FAKE + 256, None, 0)
    assert call_decode(lib, shape(T=1, L=4), content=no_sum) == INVALID
    assert call_decode(lib, shape(T=1), k=FAKE + 4) == INVALID                # misaligned vectors
    assert call_decode(lib, shape(T=1), log_g=FAKE + 4) == INVALID


def call_bwd_content(lib, s, content, dU1=None, dU2=None, ws_bytes=1 << 40, **kw):
    ptrs = {n: FAKE for n in ("q", "k", "v", "log_g", "w", "dO", "dq", "dk", "dv", "dlog_g", "db_x", "dw")}
    ptrs.update(kw)
    return lib.carve_bwd_content(ctypes.byref(s), ptrs["q"], ptrs["k"], ptrs["v"], ptrs["log_g"], ptrs["w"], None,
                                 ctypes.byref(content) if content is not None else None, ptrs["dO"], None, None,
                                 ptrs["dq"], ptrs["dk"], ptrs["dv"], ptrs["dlog_g"], ptrs["db_x"], ptrs["dw"],
                                 dU1, dU2, None, None, FAKE, ws_bytes, None)


def test_bwd_content_rejects_bad_arguments(lib):
    s = shape()
    plain = carve.carve_content(FAKE, None, None, 0, None, None)
    proj = carve.carve_content(FAKE, FAKE, FAKE, 16, None, None)
    assert call_bwd_content(lib, s, None) == INVALID                       # content is required
    assert call_bwd_content(lib, s, proj) == INVALID                       # projection needs dU1, dU2
    assert call_bwd_content(lib, s, plain, dU1=FAKE, dU2=FAKE) == INVALID  # ... and only then
    assert call_bwd_content(lib, s, plain, db_x=None) == INVALID
    assert call_bwd_content(lib, s, plain, dO=FAKE + 4) == INVALID
    assert call_bwd_content(lib, shape(L=48), plain) == UNSUPPORTED        # period not whole tiles
    need = lib.carve_bwd_content_workspace_size(ctypes.byref(s), ctypes.byref(proj))
    assert need > lib.carve_bwd_content_workspace_size(ctypes.byref(s), ctypes.byref(plain)) > 0
    assert call_bwd_content(lib, s, proj, dU1=FAKE, dU2=FAKE, ws_bytes=need - 1) == WORKSPACE
    # with the forward's per-period records the content-aware forward is not re-run: less workspace
    rec = carve.carve_content(FAKE, FAKE, FAKE, 16, None, None, FAKE, FAKE)
    need_rec = lib.carve_bwd_content_workspace_size(ctypes.byref(s), ctypes.byref(rec))
    assert 0 < need_rec < need
    half = carve.carve_content(FAKE, FAKE, FAKE, 16, None, None, None, FAKE)
    assert call_bwd_content(lib, s, half, dU1=FAKE, dU2=FAKE) == INVALID   # m_rec without z_rec


def test_logits_entry_points_reject_bad_arguments(lib):
    s = shape()
    g = carve.carve_gate_logits(FAKE, FAKE, FAKE, None, FAKE)
    call = lambda gates, **kw: lib.carve_fwd_logits(ctypes.byref(s), FAKE, FAKE, FAKE,
                                                    ctypes.byref(gates) if gates is not None else None, None,
                                                    kw.get("o", FAKE), None, FAKE, 1 << 40, None)
    assert call(None) == INVALID
    assert call(carve.carve_gate_logits(FAKE, None, FAKE, None, FAKE)) == INVALID     # A required
    assert call(carve.carve_gate_logits(FAKE + 4, FAKE, FAKE, None, FAKE)) == INVALID  # misaligned f
    assert call(g, o=None) == INVALID
    need = lib.carve_bwd_logits_workspace_size(ctypes.byref(s))
    assert need > 0

    def bwd(gates, db_x=None, ws_bytes=1 << 40):
        return lib.carve_bwd_logits(ctypes.byref(s), FAKE, FAKE, FAKE, ctypes.byref(gates), None, FAKE, None,
                                    FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, db_x, FAKE, None, FAKE, ws_bytes, None)
    assert bwd(g, db_x=FAKE) == INVALID                                                # db_x only with b_x
    assert bwd(carve.carve_gate_logits(FAKE, FAKE, FAKE, FAKE, FAKE)) == INVALID       # ... and then required
    assert bwd(g, ws_bytes=need - 1) == WORKSPACE


def test_noalloc_rejects_beyond_scratch_on_host(lib):
    """carve_fwd_noalloc checks the shape's workspace against its fixed scratch before it
    touches the device (B2 H16 T2048 d128 bf16 needs more than 64 MiB)."""
    s = shape(B=2, H=16, T=2048)
    need = lib.carve_fwd_workspace_size(ctypes.byref(s), None)
    assert need > (64 << 20)
    assert lib.carve_fwd_noalloc(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, None,
                                 None) == WORKSPACE
    # argument errors come first, as for carve_fwd
    assert lib.carve_fwd_noalloc(ctypes.byref(shape(Dv=96)), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None,
                                 FAKE, None, None) == UNSUPPORTED
    # unequal widths: the padded operands count against the scratch too
    su = shape(B=2, H=16, T=1024, D=64, Dv=128)
    assert lib.carve_fwd_workspace_size(ctypes.byref(su), None) > (64 << 20)
    assert lib.carve_fwd_noalloc(ctypes.byref(su), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE, None,
                                 None) == WORKSPACE
    c = carve.carve_content(FAKE, FAKE, FAKE, 16, None, None)
    assert lib.carve_fwd_noalloc(ctypes.byref(shape(D=64, Dv=128)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                 ctypes.byref(c), FAKE, None, None) == INVALID     # b together with content


def test_stream_copy_rejects_bad_arguments_on_host(lib):
    """The copy helper checks sizes, alignment and overlap before it touches the device;
    zero bytes is a no-op."""
    lib.carve_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    a, b = 1 << 20, 1 << 24
    assert lib.carve_stream_copy(None, None, 0, None) == 0
    assert lib.carve_stream_copy(a, b, 24, None) == INVALID        # not a multiple of 16
    assert lib.carve_stream_copy(a + 8, b, 32, None) == INVALID    # misaligned destination
    assert lib.carve_stream_copy(a, None, 32, None) == INVALID     # missing source
    assert lib.carve_stream_copy(a, a + 16, 64, None) == INVALID   # overlapping ranges


def test_size_limits_on_host(lib):
    """The largest accepted shapes and the first rejected ones: B*H is a launch grid's y
    extent (at most 65535), T at most 2^30; the workspace size of the largest head count
    is finite and nonzero."""
    assert call_fwd(lib, shape(B=5, H=13108, T=65, D=64)) == UNSUPPORTED          # B*H = 65540
    assert call_fwd(lib, shape(B=1, H=65536, T=1, D=64)) == UNSUPPORTED
    assert call_fwd(lib, shape(B=1, H=1, T=(1 << 30) + 1, D=64)) == UNSUPPORTED
    s = shape(B=5, H=13107, T=65, D=64)                                          # B*H = 65535
    ws = lib.carve_fwd_workspace_size(ctypes.byref(s), None)
    assert 0 < ws < (1 << 40)
    assert 0 < lib.carve_saved_size(ctypes.byref(s)) < (1 << 40)


def test_unequal_widths_on_host(lib):
    """Key and value widths 64 and 128 in either order run at the wider width on padded
    copies held in front of the workspace (or the saved buffer): every size grows by the
    padded operands and the checks are those of the equal-width calls."""
    for dk, dv in ((64, 128), (128, 64)):
        s, wide = shape(D=dk, Dv=dv), shape(D=128)
        for fn in ("carve_bwd_workspace_size", "carve_saved_size", "carve_bwd_saved_workspace_size"):
            assert getattr(lib, fn)(ctypes.byref(s)) > getattr(lib, fn)(ctypes.byref(wide)), fn
        need = lib.carve_fwd_workspace_size(ctypes.byref(s), None)
        assert need > lib.carve_fwd_workspace_size(ctypes.byref(wide), None)
        assert call_fwd(lib, s, ws_bytes=need - 1) == WORKSPACE
        assert call_fwd(lib, s, o=None) == INVALID
        assert call_fwd(lib, s, k=FAKE + 4) == INVALID
        assert call_bwd(lib, s, b=FAKE, db=None) == INVALID
        assert call_bwd(lib, s, ws_bytes=lib.carve_bwd_workspace_size(ctypes.byref(s)) - 1) == WORKSPACE
        c = carve.carve_content(FAKE, FAKE, FAKE, 16, None, None)
        cw = lib.carve_fwd_workspace_size(ctypes.byref(wide), ctypes.byref(c))
        assert lib.carve_fwd_workspace_size(ctypes.byref(s), ctypes.byref(c)) > cw    # content operands padded too
        assert call_fwd(lib, s, content=c, ws_bytes=cw) == WORKSPACE
        assert call_fwd(lib, s, b=FAKE, content=c) == INVALID                         # b together with content
        assert call_fwd(lib, shape(D=dk, Dv=dv, L=16), content=c) == UNSUPPORTED      # period not whole tiles
        assert lib.carve_bwd_content_workspace_size(ctypes.byref(s), ctypes.byref(c)) > \
            lib.carve_bwd_content_workspace_size(ctypes.byref(wide), ctypes.byref(c))
        for fn in ("carve_bwd_logits_workspace_size", "carve_bwd_logits_saved_workspace_size"):
            assert getattr(lib, fn)(ctypes.byref(s)) > getattr(lib, fn)(ctypes.byref(wide)), fn
        # an empty problem needs no workspace and launches nothing
        s0 = shape(T=0, D=dk, Dv=dv)
        assert lib.carve_fwd_workspace_size(ctypes.byref(s0), None) == 0
        assert call_fwd(lib, s0, q=None, k=None, v=None, log_g=None, w=None, o=None, ws=None, ws_bytes=0) == OK
