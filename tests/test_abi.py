"""The C ABI on the host: the library loads, exports what the header declares,
and rejects bad arguments synchronously (no GPU needed: these paths never
reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


@pytest.fixture(scope="module")
def lib():
    from rejection_sampling_verification_sv_amd import specverify as b
    if not os.path.exists(b.LIB_PATH):
        from rejection_sampling_verification_sv_amd import build
        build.build()
    return b.library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = _declared()
    for n in ("sv_verify_chain", "sv_verify_tree_greedy", "sv_build_tree_mask"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in enumerate(["SV_OK", "SV_ERR_INVALID_ARGUMENT", "SV_ERR_UNSUPPORTED", "SV_ERR_WORKSPACE",
                                 "SV_ERR_HIP"]):
        assert lib.sv_status_string(code).decode() == name
    assert lib.sv_status_string(99).decode() == "SV_ERR_UNKNOWN"


def test_workspace_sizes(lib):
    assert lib.sv_chain_workspace_bytes(64, 5, 128256, 1) > 0
    assert lib.sv_chain_workspace_bytes(64, 64, 128256, 1) == 0   # K > 63
    assert lib.sv_chain_workspace_bytes(64, 5, 0, 1) == 0         # V < 1
    assert lib.sv_chain_workspace_bytes(-1, 5, 10, 1) == 0
    assert lib.sv_chain_workspace_bytes(4, 4, 10, 7) == 0         # bad dtype
    assert lib.sv_tree_workspace_bytes(32, 64, 128256, 1) > 0
    assert lib.sv_tree_workspace_bytes(32, 1025, 128256, 1) == 0
    assert lib.sv_tree_workspace_bytes(32, 0, 128256, 1) == 0
    # grows with the batch
    assert lib.sv_chain_workspace_bytes(128, 5, 128256, 1) > lib.sv_chain_workspace_bytes(64, 5, 128256, 1)


def test_workspace_sizes_every_row_width(lib):
    # rows narrower than, equal to and just past one 16-byte vector, and wide
    # ones: the host layout arithmetic holds for every width
    for dt in (0, 1):
        for V in list(range(1, 41)) + [127, 128, 129, 32000, 128256, 152064, 256000]:
            for B, K in ((1, 0), (7, 1), (64, 5), (1024, 8)):
                assert lib.sv_chain_workspace_bytes(B, K, V, dt) > 0, (B, K, V, dt)
            assert lib.sv_tree_workspace_bytes(32, 64, V, dt) > 0, (V, dt)


FAKE = 0x10000  # a non-NULL address that is never dereferenced on these paths


def _chain(lib, **kw):
    a = dict(t=FAKE, d=FAKE, dt=1, x=FAKE, T=None, u=FAKE, B=4, K=4, V=100, acc=FAKE, out=FAKE,
             p=None, q=None, s=None, h=None, err=None, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.sv_verify_chain(a["t"], a["d"], a["dt"], a["x"], a["T"], a["u"], a["B"], a["K"], a["V"],
                               a["acc"], a["out"], a["p"], a["q"], a["s"], a["h"], a["err"], a["ws"], a["wsb"],
                               a["stream"])


def test_chain_argument_errors(lib):
    from rejection_sampling_verification_sv_amd import specverify as b
    b._load()
    INV, WS = 1, 3
    assert _chain(lib, t=None) == INV
    assert _chain(lib, u=None) == INV
    assert _chain(lib, acc=None) == INV
    assert _chain(lib, out=None) == INV
    assert _chain(lib, d=None) == INV            # K > 0 needs draft logits
    assert _chain(lib, x=None) == INV
    assert _chain(lib, K=64) == INV
    assert _chain(lib, V=0) == INV
    assert _chain(lib, B=-1) == INV
    assert _chain(lib, dt=5) == INV
    assert _chain(lib, t=FAKE + 1) == INV        # misaligned bf16 logits
    assert _chain(lib, ws=None) == WS
    assert _chain(lib, wsb=16) == WS
    assert _chain(lib, B=0, t=None) == 0          # empty batch: nothing to do


def test_tree_and_mask_argument_errors(lib):
    INV, WS = 1, 3
    f = lib.sv_verify_tree_greedy
    args = [FAKE, 1, FAKE, FAKE, 4, 8, 100, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None]
    assert f(*args[:2], None, *args[3:]) == INV
    bad_n = list(args)
    bad_n[5] = 1025
    assert f(*bad_n) == INV
    small = list(args)
    small[12] = 8
    assert f(*small) == WS
    assert lib.sv_build_tree_mask(None, 4, FAKE, None, None) == INV
    assert lib.sv_build_tree_mask(FAKE, 0, FAKE, None, None) == INV
    assert lib.sv_build_tree_mask(FAKE, 1025, FAKE, None, None) == INV


def test_tree_sampling_argument_errors(lib):
    INV, UNS, WS = 1, 2, 3
    f = lib.sv_verify_tree_sampling

    def call(**kw):
        a = dict(t=FAKE, d=FAKE, dt=1, x=FAKE, par=FAKE, T=None, u=FAKE, B=4, N=8, V=128, acc=FAKE, path=FAKE,
                 nxt=FAKE, err=None, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return f(a["t"], a["d"], a["dt"], a["x"], a["par"], a["T"], a["u"], a["B"], a["N"], a["V"], a["acc"],
                 a["path"], a["nxt"], a["err"], a["ws"], a["wsb"], None)
    assert call(t=None, d=None, x=None, par=None, u=None, acc=None, path=None, nxt=None, ws=None, B=0) == 0
    for k in ("t", "d", "x", "par", "u", "acc", "path", "nxt"):
        assert call(**{k: None}) == INV, k
    assert call(N=0) == INV and call(N=1025) == INV and call(V=0) == INV and call(B=-1) == INV
    assert call(dt=5) == INV
    assert call(t=FAKE + 1) == INV and call(d=FAKE + 1) == INV      # not element-aligned
    assert call(ws=None) == WS and call(wsb=16) == WS
    # valid but outside the one-pass walk: rows off 16-byte boundaries, more
    # than 1024 runs of 128 vectors per row
    assert call(V=100) == UNS
    assert call(t=FAKE + 2) == UNS and call(d=FAKE + 2) == UNS
    assert call(B=1, N=1, V=1048584) == UNS
    # at least one 8-byte record per row of the 2 B (N+1) target and draft rows,
    # and two 8-byte exchange slots per run of 128 vectors of each sequence
    for B, N, V, dt in ((32, 64, 128256, 1), (1, 1, 8, 1), (3, 5, 1000, 0)):
        ws = lib.sv_tree_sampling_workspace_bytes(B, N, V, dt)
        nrun = -(-(V * (2 if dt else 4) // 16) // 128)
        assert ws >= 8 * 2 * B * (N + 1) + 8 * 2 * B * nrun
    assert lib.sv_tree_sampling_workspace_bytes(4, 0, 128, 1) == 0
    assert lib.sv_tree_sampling_workspace_bytes(4, 8, 128, 9) == 0


def test_sample_argument_errors(lib):
    def call(**kw):
        a = dict(x=FAKE, dt=1, T=None, u=FAKE, R=4, V=100, out=FAKE, p=None, err=None, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return lib.sv_sample_rows(a["x"], a["dt"], a["T"], a["u"], a["R"], a["V"], a["out"], a["p"], a["err"],
                                  a["ws"], a["wsb"], None)
    assert call(x=None, u=None, out=None, ws=None, R=0) == 0      # nothing to do
    assert call(x=None) == 1 and call(u=None) == 1 and call(out=None) == 1
    assert call(dt=5) == 1 and call(V=0) == 1 and call(R=-1) == 1
    assert call(ws=None) == 3 and call(wsb=16) == 3
    # the sampling workspace covers the K = 0 chain layout (rows off 16-byte
    # boundaries) and one 8-byte record per run of 128 vectors (aligned rows)
    for R, V, dt in ((320, 128256, 1), (2048, 152064, 1), (5, 600000, 1), (7, 4099, 1), (16, 32000, 0)):
        ws = lib.sv_sample_workspace_bytes(R, V, dt)
        assert ws >= lib.sv_chain_workspace_bytes(R, 0, V, dt)
        if (V * (2 if dt else 4)) % 16 == 0:
            assert ws >= 8 * R * -(-(V * (2 if dt else 4) // 16) // 128)
    assert lib.sv_sample_workspace_bytes(4, 0, 1) == 0


def test_stream_pass_hook_arguments(lib):
    INV = 1
    f = lib.sv_time_next_stream_pass
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert f(FAKE, None) == INV
    assert f(None, FAKE) == INV
    # arming and disarming touch no event (the handles are only used at launch)
    assert f(FAKE, FAKE + 64) == 0
    assert f(None, None) == 0
    # a call that fails its argument checks also disarms the hook
    assert f(FAKE, FAKE + 64) == 0
    assert _chain(lib, t=None) == INV
    assert f(None, None) == 0


def test_chain_launches_query(lib):
    # host-only query of the launch form; without a device the library
    # cannot size the grid against one and answers 2 where one launch needs it
    f = lib.sv_chain_launches
    f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int, ctypes.c_int32, ctypes.c_int32]
    f.restype = ctypes.c_int32
    assert f(-1, 5, 10, 1, 1, 0) == 0 and f(4, 64, 10, 1, 1, 0) == 0 and f(4, 2, 0, 1, 1, 0) == 0
    assert f(4, 2, 10, 7, 1, 0) == 0      # bad dtype
    assert f(0, 5, 128256, 1, 1, 0) == 0  # nothing to launch
    assert f(64, 5, 128256, 1, 1, 1) in (1, 2)  # entropy: its own one-launch kernel
    assert f(64, 5, 128255, 1, 1, 0) == 2  # rows off 16-byte boundaries
    assert f(64, 0, 128256, 1, 1, 0) == 2  # K = 0
    assert f(64, 5, 128256, 1, 1, 0) in (1, 2)


def test_chain_form_query(lib):
    # host-only; without a device the call cannot be sized against one, so
    # only the two-launch form (3) is reported for valid shapes
    f = lib.sv_chain_form
    f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int, ctypes.c_int32, ctypes.c_int32]
    f.restype = ctypes.c_int32
    assert f(-1, 5, 10, 1, 1, 0) == 0 and f(4, 2, 10, 7, 1, 0) == 0 and f(0, 5, 128256, 1, 1, 0) == 0
    assert f(4, 4, 32000, 0, 1, 1) == 3      # entropy requested: never the small form (and too small for one launch)
    assert f(4, 4, 32000, 0, 0, 0) == 3      # rows off 16-byte boundaries
    assert f(4, 0, 32000, 0, 1, 0) == 3      # K = 0
    assert f(4, 4, 32000, 0, 1, 0) in (1, 3)


def test_noalloc_rejects_oversize_before_touching_the_device(lib):
    # B=256 K=63 V=256000 bf16 needs more workspace than the static array
    # holds: rejected from the sizes alone (no pointer is dereferenced)
    f = lib.sv_verify_chain_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 8
    ws = lib.sv_chain_workspace_bytes
    ws.restype = ctypes.c_size_t
    ws.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
    assert ws(256, 63, 256000, 1) > 8 << 20 >= ws(1024, 6, 256000, 1)
    fake = ctypes.c_void_p(16)  # never dereferenced on these paths
    assert f(None, None, 1, None, None, None, 256, 63, 256000, fake, None, None, None, None, None, None, None) == 2
    assert f(None, None, 1, None, None, None, 4, 64, 100, fake, None, None, None, None, None, None, None) == 1
    assert f(None, None, 1, None, None, None, 0, 5, 100, fake, None, None, None, None, None, None, None) == 0
