"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/delta.h declares, and rejects bad arguments with the documented codes before
enqueuing any work.  No call here reaches a kernel launch."""
import ctypes
import os

import pytest

import chunkwise_delta_rule_chunked_amd as D

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(D.lib_path()):
        pytest.fail("libdelta.so is not built (run `python -m chunkwise_delta_rule_chunked_amd.build`)")
    return D.load_library()


def test_exports_every_header_function(lib):
    names = D.header_functions()
    assert set(names) == {"delta_fwd_workspace_bytes", "delta_fwd", "delta_fwd_noalloc", "delta_fwd_intra", "delta_fwd_inter",
                          "delta_fwd_segments", "delta_fwd_scan_summary", "delta_fwd_scan_combine",
                          "delta_fwd_scan_outputs", "delta_chunk_wy", "delta_decode", "delta_decode_kda", "delta_fwd_kda",
                          "delta_fwd_kda_chunked", "delta_fwd_kda_chunked_workspace_bytes",
                          "delta_bwd_workspace_bytes", "delta_bwd", "delta_layer_prologue", "delta_layer_prologue_step",
                          "delta_layer_epilogue", "delta_strerror"}
    for n in names:
        assert hasattr(lib, n), n


def test_measure_header_exported(lib):
    names = D.header_functions(os.path.join(ROOT, "include", "delta_measure.h"))
    assert names == ["delta_measure_copy"] and hasattr(lib, "delta_measure_copy")
    # argument checks come before any device call
    assert lib.delta_measure_copy(None, None, 0, 4, 16, 0, None) == 0
    assert lib.delta_measure_copy(None, fake(1), 64, 4, 16, 0, None) == -1
    assert lib.delta_measure_copy(fake(0), fake(1), 40, 4, 16, 0, None) == -4
    assert lib.delta_measure_copy(fake(0), fake(1), 64, 3, 16, 0, None) == -3
    assert lib.delta_measure_copy(fake(0), ctypes.c_void_p(A + 32), 64, 4, 16, 0, None) == -6


def test_strerror(lib):
    for code in range(0, -10, -1):
        msg = D.strerror(code)
        assert msg and msg != "unknown error code", code
    assert D.strerror(-99) == "unknown error code"


def shape(**kw):
    base = dict(B=2, L=100, H=3, dk=64, dv=32, n_h=1, chunk=32, dtype=D.BF16, scale=1.0)
    base.update(kw)
    return D.make_shape(**base)


def ws(sh):
    n = ctypes.c_size_t(0)
    rc = D.load_library().delta_fwd_workspace_bytes(ctypes.byref(sh), ctypes.byref(n))
    return rc, n.value


def segments(B, H, dv, NT):
    """Sequence split of the inter-chunk pass: about 256 output workgroups in total (4 or 8
    state column tiles per workgroup), each segment at least one chunk."""
    tiles = 4 if dv <= 64 else 8
    units = B * H * (-(-(dv // 16) // tiles))
    P = 256 // units if units > 0 and NT > 1 else 1
    P = max(1, min(P, NT if NT > 0 else 1))
    NS = -(-NT // P) if NT > 0 else 1
    return (-(-NT // NS) if NT > 0 else 1), NS


def test_segments_rule():
    assert segments(2, 16, 128, 128) == (8, 16)     # 32 heads: 8 segments of 16 chunks
    assert segments(1, 16, 128, 1024) == (16, 64)
    assert segments(4, 8, 128, 32) == (8, 4)
    assert segments(64, 16, 128, 4) == (1, 4)       # enough heads: no split
    assert segments(1, 1, 16, 4) == (4, 1)
    assert segments(1, 1, 16, 5) == (5, 1)
    assert segments(2, 1, 16, 300) == (100, 3)      # 128 wanted; segments of 3 chunks -> 100
    assert segments(2, 1, 16, 300)[0] * segments(2, 1, 16, 300)[1] >= 300


def test_segments_reported(lib):
    for B, H, L, dv, C in [(2, 16, 8192, 128, 64), (1, 16, 65536, 128, 64), (4, 8, 2048, 128, 64),
                           (64, 16, 64, 128, 64), (1, 1, 64, 16, 16), (2, 3, 100, 32, 32), (1, 1, 0, 16, 16)]:
        NT = (L + C - 1) // C
        assert D.segments(B, L, H, 128 if dv == 128 else 64, dv, 1, C) == segments(B, H, dv, NT), (B, H, L, dv, C)


def test_workspace_bytes(lib):
    up = lambda x: (x + 255) // 256 * 256
    for B, H, L, dk, dv, C, dt, es in [(2, 3, 100, 64, 32, 32, D.BF16, 2), (2, 3, 100, 64, 32, 32, D.F32, 4),
                                       (2, 16, 8192, 128, 128, 64, D.BF16, 2), (64, 16, 64, 128, 128, 64, D.BF16, 2),
                                       (1, 1, 50, 16, 256, 16, D.F32, 4)]:
        rc, n = ws(shape(B=B, H=H, L=L, dk=dk, dv=dv, chunk=C, dtype=dt))
        NT = (L + C - 1) // C
        P, _ = segments(B, H, dv, NT)
        t_bytes = B * H * NT * C * C * es
        gc_bytes = B * H * NT * C * 4
        seg = up(B * H * P * dk * (dv + dk) * 4) + up(B * H * P * dk * dv * 4) if P > 1 else 0
        assert rc == 0 and n == up(t_bytes) + up(gc_bytes) + seg, (B, H, L, dk, dv, C)
    assert ws(shape(L=0)) == (0, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=48), -3), (dict(dk=256), -3), (dict(dv=8), -3), (dict(dv=40), -3), (dict(dv=272), -3),
    (dict(chunk=24), -3), (dict(chunk=128), -3), (dict(dtype=7), -3),
    (dict(n_h=0), -2), (dict(B=-1), -2), (dict(L=-5), -2), (dict(n_h=3, chunk=32), -2),
])
def test_shape_errors(lib, kw, code):
    assert ws(shape(**kw))[0] == code


# Fake, never-dereferenced device addresses: every call below fails validation first.  As a
# guard against a validation slip reaching a launch with them, these run only without a GPU.
A = 1 << 20


@pytest.fixture
def no_gpu():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("fake-pointer argument checks run on hosts without a GPU")


def fake(i):
    return ctypes.c_void_p(A * (i + 1))


def call_fwd(sh, q=None, k=None, v=None, beta=None, g=None, S0=None, O=None, SF=None, w=None, wbytes=None):
    args = [fake(0) if q is None else q, fake(1) if k is None else k, fake(2) if v is None else v,
            fake(3) if beta is None else beta, g, S0, fake(4) if O is None else O, SF,
            fake(5) if w is None else w]
    if wbytes is None:
        wbytes = ws(sh)[1]
    return D.load_library().delta_fwd(ctypes.byref(sh), *args, ctypes.c_size_t(wbytes), None)


def test_fwd_argument_errors(lib, no_gpu):
    sh = shape()
    big = ctypes.c_void_p(0)
    assert call_fwd(sh, q=big) == -1                    # q NULL
    assert call_fwd(sh, beta=big) == -1                 # beta NULL
    assert call_fwd(sh, w=big) == -5                    # workspace NULL
    assert call_fwd(sh, wbytes=ws(sh)[1] - 1) == -5     # workspace too small
    assert call_fwd(sh, k=ctypes.c_void_p(A * 2 + 8)) == -4   # misaligned
    assert call_fwd(sh, O=fake(0)) == -6                # O aliases q
    assert call_fwd(sh, w=fake(2)) == -6                # workspace aliases v
    # S_final partially overlapping S0 is an error; in-place (equal) passes this check but
    # must then fail elsewhere here: make O alias q to stop before launching
    S0 = ctypes.c_void_p(A * 40)
    assert call_fwd(sh, S0=S0, SF=ctypes.c_void_p(A * 40 + 256)) == -6
    assert call_fwd(sh, S0=S0, SF=S0, O=fake(0)) == -6
    assert call_fwd(shape(n_h=5, chunk=48)) == -2       # chunk not a multiple of n_h


def test_decode_argument_errors(lib, no_gpu):
    L = D.load_library()
    sh = shape(L=2)
    f = [fake(i) for i in range(7)]
    assert L.delta_decode(ctypes.byref(sh), *f[:5], f[5], f[6], None) == -2          # L != 1
    sh = shape(L=1)
    assert L.delta_decode(ctypes.byref(sh), None, *f[1:5], f[5], f[6], None) == -1   # q NULL
    assert L.delta_decode(ctypes.byref(sh), *f[:5], f[0], f[6], None) == -6          # S aliases q
    assert L.delta_decode(ctypes.byref(sh), *f[:5], ctypes.c_void_p(A * 6 + 4), f[6], None) == -4


def test_decode_kda_argument_errors(lib, no_gpu):
    L = D.load_library()
    f = [fake(i) for i in range(7)]
    sh = shape(L=1)
    assert L.delta_decode_kda(ctypes.byref(sh), *f[:4], None, f[5], f[6], None) == -1    # a_log NULL
    assert L.delta_decode_kda(ctypes.byref(shape(L=1, n_h=2, chunk=64)), *f[:5], f[5], f[6], None) == -2
    assert L.delta_decode_kda(ctypes.byref(shape(L=2)), *f[:5], f[5], f[6], None) == -2   # L != 1
    assert L.delta_decode_kda(ctypes.byref(sh), *f[:4], f[5], f[5], f[6], None) == -6     # a_log aliases S
    assert L.delta_decode_kda(ctypes.byref(sh), *f[:4], ctypes.c_void_p(A * 4 + 2), f[5], f[6], None) == -4
    assert L.delta_decode_kda(ctypes.byref(shape(B=0, L=1)), *[None] * 7, None) == 0       # empty


def bwd_ws(sh):
    n = ctypes.c_size_t(0)
    rc = D.load_library().delta_bwd_workspace_bytes(ctypes.byref(sh), ctypes.byref(n))
    return rc, n.value


def test_bwd_workspace_bytes(lib):
    """Vector-ALU scans: T and Q K^T * Gam (float32, C x C per chunk), the gate prefix and two
    float32 states per chunk.  State scans on the inter-chunk machinery (bf16, d_k = d_v = 128,
    chunk 64): T (bf16), the gate prefix, N (float32), the segment summaries and start states,
    and per chunk the start state (bf16) and the end-state gradient (bf16 high and low parts)."""
    up = lambda x: (x + 255) // 256 * 256
    for B, H, L, dk, dv, C, nh, dt in [(2, 3, 100, 64, 32, 32, 1, D.BF16), (2, 16, 8192, 128, 128, 64, 1, D.F32),
                                       (1, 2, 50, 16, 256, 48, 3, D.BF16), (2, 16, 8192, 128, 128, 64, 1, D.BF16),
                                       (1, 2, 300, 128, 128, 64, 2, D.BF16), (64, 16, 100, 128, 128, 64, 1, D.BF16)]:
        NT = (L * nh + C - 1) // C
        rc, n = bwd_ws(shape(B=B, H=H, L=L, dk=dk, dv=dv, chunk=C, n_h=nh, dtype=dt))
        states = B * H * NT * dk * dv * 4
        if dt == D.BF16 and dk == dv == 128 and C == 64:
            P, _ = segments(B, H, dv, NT)
            sm = B * H * P * dk * (dv + dk) * 4 if P > 1 else 0
            sst = B * H * P * dk * dv * 4 if P > 1 else 0
            want = (up(B * H * NT * C * C * 2) + up(B * H * NT * C * 4) + up(B * H * NT * C * C * 4) + 2 * up(sm) + up(sst)
                    + 3 * up(states // 2))
        else:
            want = 2 * up(B * H * NT * C * C * 4) + up(B * H * NT * C * 4) + 2 * up(states)
        assert rc == 0 and n == want, (B, H, L, dk, dv, C, nh, dt)
    assert bwd_ws(shape(L=0)) == (0, 0)
    assert bwd_ws(shape(dk=48))[0] == -3


def call_bwd(sh, **kw):
    names = ["q", "k", "v", "beta", "g", "S0", "dO", "dSF", "dq", "dk", "dv", "dbeta", "dg", "dS0", "w"]
    defaults = {"q": 0, "k": 1, "v": 2, "beta": 3, "dO": 4, "dq": 5, "dk": 6, "dv": 7, "dbeta": 8, "w": 9}
    args = [kw[n] if n in kw else (fake(defaults[n]) if n in defaults else None) for n in names]
    wbytes = kw.get("wbytes", bwd_ws(sh)[1])
    return D.load_library().delta_bwd(ctypes.byref(sh), *args, ctypes.c_size_t(wbytes), None)


def test_bwd_argument_errors(lib, no_gpu):
    sh = shape()
    assert call_bwd(sh, dO=None) == -1                      # dO NULL
    assert call_bwd(sh, dbeta=None) == -1                   # dbeta NULL
    assert call_bwd(sh, w=None) == -5                       # workspace NULL
    assert call_bwd(sh, wbytes=bwd_ws(sh)[1] - 1) == -5     # workspace too small
    assert call_bwd(sh, dk=ctypes.c_void_p(A * 7 + 8)) == -4  # misaligned
    assert call_bwd(sh, dq=fake(0)) == -6                   # dq aliases q
    assert call_bwd(sh, dv=fake(6)) == -6                   # dv aliases dk
    assert call_bwd(sh, dS0=fake(9)) == -6                  # dS0 inside the workspace
    assert call_bwd(shape(chunk=24)) == -3
    assert D.load_library().delta_bwd(ctypes.byref(shape(B=0)), *[None] * 15, ctypes.c_size_t(0), None) == 0


def test_layer_argument_errors(lib, no_gpu):
    L = D.load_library()
    sh = shape()
    f = [fake(i) for i in range(9)]
    assert L.delta_layer_prologue(ctypes.byref(sh), 5, ctypes.c_float(1e-6), *f, None) == -3     # width
    assert L.delta_layer_prologue(ctypes.byref(sh), 4, ctypes.c_float(-1.0), *f, None) == -2     # eps < 0
    assert L.delta_layer_prologue(ctypes.byref(sh), 4, ctypes.c_float(1e-6), None, *f[1:], None) == -1
    assert L.delta_layer_prologue(ctypes.byref(sh), 4, ctypes.c_float(1e-6), *f[:6], f[0], f[7], f[8], None) == -6
    assert L.delta_layer_prologue(ctypes.byref(sh), 4, ctypes.c_float(1e-6), *f[:8], ctypes.c_void_p(A * 9 + 4), None) == -4
    assert L.delta_layer_epilogue(ctypes.byref(sh), ctypes.c_float(1e-6), f[0], f[1], f[2], f[1], None) == -6  # y aliases g
    assert L.delta_layer_epilogue(ctypes.byref(sh), ctypes.c_float(1e-6), f[0], None, f[2], f[3], None) == -1
    assert L.delta_layer_epilogue(ctypes.byref(shape(B=0)), ctypes.c_float(1e-6), None, None, None, None, None) == 0


def test_chunk_wy_argument_errors(lib, no_gpu):
    L = D.load_library()
    sh = shape()
    f = [fake(i) for i in range(8)]
    assert L.delta_chunk_wy(ctypes.byref(sh), None, f[1], f[2], None, f[3], None, None, f[4], None) == -1
    assert L.delta_chunk_wy(ctypes.byref(sh), f[0], f[1], f[2], None, f[0], None, None, f[4], None) == -6
    assert L.delta_chunk_wy(ctypes.byref(shape(chunk=20)), *f[:3], None, f[3], None, None, f[4], None) == -3


def test_empty_problems_are_noops(lib, no_gpu):
    # B = 0 or H = 0: nothing to compute, no pointers needed, returns OK without launching
    sh = shape(B=0)
    assert D.load_library().delta_fwd(ctypes.byref(sh), *[None] * 9, ctypes.c_size_t(0), None) == 0
    sh = shape(H=0, L=1)
    assert D.load_library().delta_decode(ctypes.byref(sh), *[None] * 7, None) == 0


def test_binding_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 16, 1, 16)
    with pytest.raises(ValueError):
        D.fwd(q, q, q, torch.zeros(1, 16, 1), chunk=16)


def test_fault_injection_returns_hip_error(lib, no_gpu, monkeypatch):
    """DELTA_FAULT=launch: a call that passes every argument check returns DELTA_ERR_HIP (-7) in
    place of its first launch, so callers' error paths can be tested without a GPU; calls with
    nothing to enqueue still succeed and argument errors keep their own codes."""
    monkeypatch.setenv("DELTA_FAULT", "launch")
    Lb = D.load_library()
    assert call_fwd(shape()) == -7
    assert call_fwd(shape(L=0), w=ctypes.c_void_p(0), wbytes=0, O=ctypes.c_void_p(0), SF=fake(6)) == -7  # S_final = S0
    assert call_fwd(shape(), q=ctypes.c_void_p(0)) == -1
    f = [fake(i) for i in range(9)]
    assert Lb.delta_decode(ctypes.byref(shape(L=1)), *f[:5], f[5], f[6], None) == -7
    assert Lb.delta_decode_kda(ctypes.byref(shape(L=1)), *f[:5], f[5], f[6], None) == -7
    assert Lb.delta_layer_prologue(ctypes.byref(shape()), 4, ctypes.c_float(1e-6), *f, None) == -7
    assert Lb.delta_layer_epilogue(ctypes.byref(shape()), ctypes.c_float(1e-6), f[0], f[1], f[2], f[3], None) == -7
    assert call_bwd(shape()) == -7
    assert Lb.delta_fwd(ctypes.byref(shape(B=0)), *[None] * 9, ctypes.c_size_t(0), None) == 0
    with pytest.raises(D.DeltaError) as e:
        D._check(-7, "delta_fwd")
    assert e.value.code == -7 and "HIP" in str(e.value)


def test_noalloc_limit(lib):
    """The binding's copy of DELTA_NOALLOC_MAX_BYTES matches the header, and a shape needing more
    workspace than that is rejected (-9) before any device call; shape errors keep their codes."""
    import re
    txt = open(os.path.join(ROOT, "include", "delta.h")).read()
    m = re.search(r"#define DELTA_NOALLOC_MAX_BYTES \((\d+)u << (\d+)\)", txt)
    assert m and D.NOALLOC_MAX_BYTES == int(m.group(1)) << int(m.group(2))
    sh = shape(B=1, H=16, L=65536, dk=128, dv=128, chunk=64)
    assert ws(sh)[1] > D.NOALLOC_MAX_BYTES
    assert D.load_library().delta_fwd_noalloc(ctypes.byref(sh), *[None] * 8, None) == -9
    assert D.load_library().delta_fwd_noalloc(ctypes.byref(shape(dk=48)), *[None] * 8, None) == -3


def test_kda_chunked_workspace_and_argument_checks(lib):
    """delta_fwd_kda_chunked takes bf16, dk = dv = 128, chunk 64, n_h = 1 only; its workspace holds T and
    Aqk's lower triangle (6 fragments of 64 lanes x 16 bytes per chunk), three bf16 tiles in the
    layout of k, the chunk decay (128 floats per chunk), and the segment summaries and start
    states."""
    up = lambda x: (x + 255) // 256 * 256
    L = D.load_library()
    for B, H, Ln in [(2, 16, 8192), (1, 2, 333), (2, 128, 70)]:
        NT = -(-Ln // 64)
        n = ctypes.c_size_t(0)
        assert L.delta_fwd_kda_chunked_workspace_bytes(ctypes.byref(shape(B=B, H=H, L=Ln, dk=128, dv=128, chunk=64)),
                                                       ctypes.byref(n)) == 0
        P, _ = segments(B, H, 128, NT)
        sm = B * H * P * 128 * 256 * 4 if P > 1 else 0
        sst = B * H * P * 128 * 128 * 4 if P > 1 else 0
        want = (up(B * H * NT * 64 * 64 * 2) + up(B * H * NT * 6 * 64 * 16) + 3 * up(B * Ln * H * 128 * 2)
                + up(B * H * NT * 128 * 4) + up(sm) + up(sst))
        assert n.value == want, (B, H, Ln)
    n = ctypes.c_size_t(0)
    for bad in (dict(dk=64), dict(dv=64), dict(chunk=32), dict(n_h=2, chunk=64), dict(dtype=D.F32)):
        kw = dict(B=1, H=2, L=100, dk=128, dv=128, chunk=64)
        kw.update(bad)
        assert L.delta_fwd_kda_chunked_workspace_bytes(ctypes.byref(shape(**kw)), ctypes.byref(n)) == -3, bad
    sh = shape(B=1, H=2, L=100, dk=128, dv=128, chunk=64)
    f = [ctypes.c_void_p(4096 * (i + 1) * 1024) for i in range(9)]
    args = f[:5] + [None] + f[5:7]                        # q k v beta a_log S0 O S_final
    assert L.delta_fwd_kda_chunked(ctypes.byref(sh), *args, f[8], ctypes.c_size_t(16), None) == -5   # workspace small
    assert L.delta_fwd_kda_chunked(ctypes.byref(sh), *args, None, ctypes.c_size_t(0), None) == -5
    big = ctypes.c_size_t(1 << 40)
    assert L.delta_fwd_kda_chunked(ctypes.byref(sh), *args, f[0], big, None) == -6                     # aliases q
    assert L.delta_fwd_kda_chunked(ctypes.byref(sh), f[0], None, *args[2:], f[8], big, None) == -1     # k NULL
    assert L.delta_fwd_kda_chunked(ctypes.byref(shape(B=1, H=2, L=100, dk=64, dv=64, chunk=64)), *args, f[8], big,
                                   None) == -3
