"""Host-side checks of the C ABI: the library loads, exports every function
include/falcon.h declares, and rejects malformed arguments with the
documented status before launching anything.  No GPU needed."""
from __future__ import annotations

import ctypes
import pathlib
import re

import pytest

from linear_recurrent_weight_amd import falcon as fb

ROOT = pathlib.Path(__file__).resolve().parent.parent


@pytest.fixture(scope="module")
def lib():
    if not fb.LIB_PATH.exists():
        pytest.skip("libfalcon.so not built")
    return fb.load_library()


def header_functions():
    text = (ROOT / "include" / "falcon.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(falcon_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert header_functions() == sorted(fb.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.falcon_abi_version() == fb.ABI_VERSION


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, 7):
        assert isinstance(lib.falcon_status_str(st), bytes)
    assert lib.falcon_status_str(-3) == b"workspace missing or too small"


FAKE = 1 << 20  # an aligned, never dereferenced address


def args(**kw):
    base = dict(variant="F1", dtype="bf16", batch=2, heads=3, seqlen=128, dk=64, dv=64, chunk=64,
                window=1, q=FAKE, k=2 * FAKE, v=3 * FAKE, beta=4 * FAKE, lam=5 * FAKE, o=6 * FAKE)
    base.update(kw)
    return fb.make_args(**base)


def validate(lib, a):
    return lib.falcon_fwd_validate(ctypes.byref(a))


def wsize(lib, a):
    return lib.falcon_fwd_workspace_size(ctypes.byref(a))


def _align(n):
    return -(-n // 256) * 256


def with_ws(lib, a):
    n = wsize(lib, a)
    a.workspace = 1 << 30
    a.workspace_bytes = n
    return a


def test_valid_arguments(lib):
    for var, w in [("F1", 1), ("F2", 1), ("F3", 4), ("F1A", 1), ("F3A", 8)]:
        a = with_ws(lib, args(variant=var, window=w, chunk=0))
        assert validate(lib, a) == fb.OK, var
    assert validate(lib, with_ws(lib, args())) == fb.OK


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 99, fb.ERR_INVALID_ARG),
    ("variant", 4, fb.ERR_INVALID_ARG),
    ("variant", 14, fb.ERR_INVALID_ARG),
    ("dtype", 2, fb.ERR_INVALID_ARG),
    ("phi", 5, fb.ERR_INVALID_ARG),
    ("batch", 0, fb.ERR_INVALID_ARG),
    ("heads", -1, fb.ERR_INVALID_ARG),
    ("seqlen", -5, fb.ERR_INVALID_ARG),
    ("dk", 48, fb.ERR_UNSUPPORTED),
    ("dv", 256, fb.ERR_UNSUPPORTED),
    ("chunk", -1, fb.ERR_INVALID_ARG),
    ("chunk", 48, fb.ERR_UNSUPPORTED),
    ("window", 0, fb.ERR_INVALID_ARG),
    ("window", 2, fb.ERR_INVALID_ARG),
    ("eps", -1.0, fb.ERR_INVALID_ARG),
    ("eps", float("nan"), fb.ERR_INVALID_ARG),
    ("eps_rms", float("inf"), fb.ERR_INVALID_ARG),
    ("eps_gamma", 0.0, fb.ERR_INVALID_ARG),
    ("eps_gamma", 1.0, fb.ERR_INVALID_ARG),
])
def test_field_rules(lib, field, value, status):
    a = with_ws(lib, args())
    setattr(a, field, value)
    assert validate(lib, a) == status
    # falcon_fwd reports the same status and launches nothing
    assert lib.falcon_fwd(ctypes.byref(a), None) == status


def test_window_limits(lib):
    a = with_ws(lib, args(variant="F3A", window=9, chunk=0))
    assert validate(lib, a) == fb.ERR_UNSUPPORTED
    a = with_ws(lib, args(variant="F3A", window=8, chunk=0))
    assert validate(lib, a) == fb.OK


@pytest.mark.parametrize("name", ["q", "k", "v", "beta", "lambda_", "o"])
def test_null_and_misaligned_tensors(lib, name):
    a = with_ws(lib, args())
    setattr(a, name, None)
    assert validate(lib, a) == fb.ERR_INVALID_ARG
    a = with_ws(lib, args())
    setattr(a, name, FAKE * 7 + 2)
    assert validate(lib, a) == fb.ERR_INVALID_ARG


def test_empty_sequence_needs_no_tensors(lib):
    a = args(seqlen=0, q=None, k=None, v=None, beta=None, lam=None, o=None)
    assert wsize(lib, a) == 0
    assert validate(lib, a) == fb.OK


def test_output_may_not_alias_inputs(lib):
    a = with_ws(lib, args(o=FAKE))
    assert validate(lib, a) == fb.ERR_INVALID_ARG


def test_workspace_rules(lib):
    a = args(dtype="f32")
    n = wsize(lib, a)
    assert n > 0
    assert validate(lib, a) == fb.ERR_WORKSPACE          # missing
    a.workspace = 1 << 30
    a.workspace_bytes = n - 1
    assert validate(lib, a) == fb.ERR_WORKSPACE          # too small
    a.workspace_bytes = n
    assert validate(lib, a) == fb.OK
    a.workspace = (1 << 30) + 64
    assert validate(lib, a) == fb.ERR_WORKSPACE          # not 256-byte aligned


def test_workspace_grows_with_problem(lib):
    small = wsize(lib, args(seqlen=64, dtype="f32"))
    big = wsize(lib, args(seqlen=1024, dtype="f32"))
    assert 0 < small < big
    # ragged lengths round up to whole chunks on the chunk path
    assert wsize(lib, args(seqlen=65, dtype="f32")) == wsize(lib, args(seqlen=128, dtype="f32"))
    # bf16 Falcon-1 at d_k = 64, d_v = 32: the transfer-operator pair keeps
    # per-chunk operators in the workspace (d_v = 64 keeps them on chip)
    assert wsize(lib, args(seqlen=1024, dv=32)) > 0
    assert validate(lib, with_ws(lib, args(seqlen=1024, dv=32))) == fb.OK
    # a malformed request reports 0 bytes
    assert wsize(lib, args(dk=48)) == 0


def test_state_rules(lib):
    S = fb.FalconStateC(7 * FAKE, 8 * FAKE, 9 * FAKE, 10 * FAKE, 0, 0)
    a = with_ws(lib, args(state_in=S))
    assert validate(lib, a) == fb.OK
    S.x_next = None                                       # continuing needs x_next
    a = with_ws(lib, args(state_in=S))
    assert validate(lib, a) == fb.ERR_INVALID_ARG
    S.fresh = 1                                           # fresh ignores it
    a = with_ws(lib, args(state_in=S))
    assert validate(lib, a) == fb.OK
    S.n_tail = 1                                          # fresh with a tail
    a = with_ws(lib, args(state_in=S))
    assert validate(lib, a) == fb.ERR_INVALID_ARG
    W = fb.FalconStateC(7 * FAKE, 8 * FAKE, 9 * FAKE, 10 * FAKE, 4, 0)
    a = with_ws(lib, args(variant="F3A", window=4, chunk=0, state_in=W))
    assert validate(lib, a) == fb.ERR_INVALID_ARG         # n_tail > W - 1
    W.n_tail = 3
    a = with_ws(lib, args(variant="F3A", window=4, chunk=0, state_in=W))
    assert validate(lib, a) == fb.OK
    W.tail_x = None
    a = with_ws(lib, args(variant="F3A", window=4, chunk=0, state_in=W))
    assert validate(lib, a) == fb.ERR_INVALID_ARG


def test_state_out_rules(lib):
    out = fb.FalconStateC(11 * FAKE, 12 * FAKE, None, None, 0, 0)
    a = with_ws(lib, args(state_out=out))
    assert validate(lib, a) == fb.OK
    a = with_ws(lib, args(variant="F3A", window=4, chunk=0, state_out=out))
    assert validate(lib, a) == fb.ERR_INVALID_ARG         # windowed needs a tail buffer
    out.x_next = None
    a = with_ws(lib, args(state_out=out))
    assert validate(lib, a) == fb.ERR_INVALID_ARG
    # state_out may not overlap state_in
    sin = fb.FalconStateC(11 * FAKE, 13 * FAKE, None, None, 0, 0)
    out = fb.FalconStateC(11 * FAKE, 12 * FAKE, None, None, 0, 0)
    a = with_ws(lib, args(state_in=sin, state_out=out))
    assert validate(lib, a) == fb.ERR_INVALID_ARG


def test_chunk_path_coverage(lib):
    """Combinations with a chunk-parallel kernel validate; the others report
    UNSUPPORTED (and the token-recurrent form takes every variant)."""
    assert validate(lib, with_ws(lib, args(variant="F1", dk=128, dv=32))) == fb.OK
    assert validate(lib, with_ws(lib, args(variant="F1", dk=16))) == fb.ERR_UNSUPPORTED
    for var in ("F1", "F2", "F3", "F1A", "F3A"):
        w = 3 if var in ("F3", "F3A") else 1
        assert validate(lib, with_ws(lib, args(variant=var, window=w, chunk=0, dk=16, dv=16))) == fb.OK


def test_f1_bf16_workspace(lib):
    """bf16 Falcon-1 at d_k = 64 (transfer operators, then the carry) keeps
    A, G, B^T and H in bf16 plus one 256-byte scalar block per chunk."""
    for dv in (32, 64, 128):
        per_chunk = 2 * 64 * 64 * 2 + 2 * 64 * dv * 2 + 256
        assert wsize(lib, args(seqlen=1000, dv=dv)) == 6 * 16 * per_chunk
        assert _names(lib, args(seqlen=1000, dv=dv)) == ["f1_xfer", "f1_carry"]


def _f1_segments(bh, dv, nchunks):
    """Chunks per segment of the bf16 Falcon-1 carry: one segment for walks
    under 48 chunks or when the carry's workgroups (32 value columns each,
    heads rounded up to 8 when a head has several) exceed 256; otherwise
    about 512 / workgroups segments of at least 16 chunks."""
    nslice = dv // min(dv, 32)
    groups = bh if nslice == 1 else -(-bh // 8) * 8 * nslice
    if nchunks < 48 or groups > 256:
        return nchunks
    return max(16, -(-nchunks // (512 // groups)))


@pytest.mark.parametrize("B,H,T,dv", [(2, 12, 16384, 64), (1, 3, 5000, 32), (1, 1, 3072, 128),
                                      (8, 12, 1024, 64), (8, 12, 16384, 64), (2, 6, 3000, 64)])
def test_f1_bf16_long_walks_split_into_segments(lib, B, H, T, dv):
    """Long walks over few heads compose each segment's chunk maps and scan
    them before the carry; the workspace adds the composed maps [A~ | beta]
    (A~ in bf16, beta in fp32), their scalars and the segments' fp32 entry
    states."""
    a = args(batch=B, heads=H, seqlen=T, dv=dv)
    bh, nch = B * H, -(-T // 64)
    g = _f1_segments(bh, dv, nch)
    nseg = -(-nch // g)
    align = lambda n: -(-n // 256) * 256
    per_chunk = 2 * 64 * 64 * 2 + 2 * 64 * dv * 2 + 256
    n = align(bh * nch * per_chunk)
    if nseg > 1:
        n += align(bh * nseg * (64 * 64 * 2 + 64 * dv * 4)) + align(bh * nseg * 4) + align(bh * nseg * 64 * dv * 4)
        assert _names(lib, a) == ["f1_xfer", "f1_segmap", "f1_segscan", "f1_carry"]
    else:
        assert _names(lib, a) == ["f1_xfer", "f1_carry"]
    assert wsize(lib, a) == n
    # the long-sequence workload with few heads is split
    if (B, H, T) == (2, 12, 16384):
        assert nseg == 10 and g == 26


@pytest.mark.parametrize("window", [2, 4, 8])
@pytest.mark.parametrize("B,H,T", [(8, 12, 512), (2, 3, 300), (1, 2, 16384)])
def test_f3_bf16_d64_transfer_path(lib, window, B, H, T):
    """bf16 Falcon-3 at d_k = d_v = 64 with W in {2, 4, 8}: the window pass,
    Falcon-1 records for every 64-token chunk and the Falcon-1 walk (split
    into segments by the Falcon-1 rule); the workspace is w_t and log2 gamma_t
    per token, the records, and the segment maps when split."""
    a = args(variant="F3", window=window, batch=B, heads=H, seqlen=T)
    bh, nch = B * H, -(-T // 64)
    g = _f1_segments(bh, 64, nch)
    nseg = -(-nch // g)
    n = 2 * _align(bh * nch * 64 * 4) + _align(bh * nch * (2 * 64 * 64 * 2 + 2 * 64 * 64 * 2 + 256))
    if nseg > 1:
        n += _align(bh * nseg * (64 * 64 * 2 + 64 * 64 * 4)) + _align(bh * nseg * 4) + _align(bh * nseg * 64 * 64 * 4)
        assert _names(lib, a) == ["a3_window", "f3_xfer", "f1_segmap", "f1_segscan", "f1_carry"]
    else:
        assert _names(lib, a) == ["a3_window", "f3_xfer", "f1_carry"]
    assert wsize(lib, a) == n
    # other windows, head sizes or fp32 keep the stacked-row kernels
    assert _names(lib, args(variant="F3", window=3, batch=B, heads=H, seqlen=T)) == ["feature", "f3_prep", "f3_scan"]
    assert _names(lib, args(variant="F3", window=window, dv=32, batch=B, heads=H, seqlen=T))[1] == "f3_prep"


def test_library_reads_no_tuning_switches():
    """Path choice, slices and segment lengths follow the arguments alone:
    the library source reads no environment variable except the debug check
    FALCON_SYNC_CHECK."""
    csrc = ROOT / "linear_recurrent_weight_amd" / "csrc"
    names = set()
    for f in list(csrc.glob("*.hip")) + list(csrc.glob("*.cpp")) + list(csrc.glob("*.h")):
        names |= set(re.findall(r'getenv\("([A-Z_]+)"\)', f.read_text()))
    assert names == {"FALCON_SYNC_CHECK"}


def test_chunk_f2_coverage(lib):
    """Falcon-2 has a chunk-parallel kernel for bf16 d_k in {64, 128} and
    fp32 d_k = 64; it needs no workspace."""
    for dt, dk, ok in [("bf16", 64, True), ("bf16", 128, True), ("f32", 64, True),
                       ("f32", 128, False), ("bf16", 32, False)]:
        a = args(variant="F2", dtype=dt, dk=dk, dv=128)
        assert validate(lib, a) == (fb.OK if ok else fb.ERR_UNSUPPORTED), (dt, dk)
        if ok:
            assert wsize(lib, a) == 0


def test_chunk_f3_coverage(lib):
    """Falcon-3 has a chunk-parallel path (stacked window rows) for every
    window; it takes workspace for features and per-chunk operators."""
    for w in (1, 2, 3, 8):
        a = args(variant="F3", window=w, dk=64, dv=64)
        n = wsize(lib, a)
        assert n > 0
        assert validate(lib, with_ws(lib, a)) == fb.OK
    assert validate(lib, with_ws(lib, args(variant="F3", window=4, dk=16))) == fb.ERR_UNSUPPORTED


def _names(lib, a):
    out = []
    while True:
        nm = lib.falcon_kernel_name(ctypes.byref(a), len(out))
        if nm is None:
            return out
        out.append(nm.decode())


def _segments(bh, nchunks):
    """Chunks per segment of the bf16 d = 64 inner-product path: the fewest
    that keep every segment of every head resident at once (512 workgroups)."""
    for g in range(1, nchunks):
        if bh * -(-nchunks // g) <= 512:
            return g
    return max(nchunks, 1)


@pytest.mark.parametrize("variant,window", [("F1A", 1), ("F3A", 2), ("F3A", 8)])
@pytest.mark.parametrize("B,H,T", [(2, 12, 16384), (8, 12, 2048)])
def test_inner_product_bf16_d64_path(lib, variant, window, B, H, T):
    """bf16 Falcon-1A / 3A at d_k = d_v = 64 take the register-transpose
    kernels (a window pass first when W > 1); their workspace is the segment
    writes and entry states (fp32 [d_k][d_v]) and carries, plus w_t and
    log2 gamma_t per token with a window.  With at most 8 segments per head
    the output walks fold their entry states themselves (no scan launch)."""
    a = args(variant=variant, window=window, batch=B, heads=H, seqlen=T)
    names = _names(lib, a)
    nch = T // 64
    g = _segments(B * H, nch)
    nseg = -(-nch // g)
    scan = ["a1_segscan"] if nseg > 8 else []
    want = (["a3_window"] if window > 1 else []) + ["a1_segment"] + scan + ["a1_output"]
    assert names == want
    assert (nseg > 8) == ((B, H, T) == (2, 12, 16384))
    align = lambda n: -(-n // 256) * 256
    st = B * H * nseg * 64 * 64 * 4
    n = align(st) + align(B * H * nseg * 4) + align(st)
    if window > 1:
        n += 2 * align(B * H * nch * 64 * 4)
    assert wsize(lib, a) == n
    # (the fake tensor addresses are 1 MiB apart: validate a small shape)
    assert validate(lib, with_ws(lib, args(variant=variant, window=window))) == fb.OK


def test_inner_product_other_shapes_take_the_general_kernels(lib):
    for dt, dk, dv in [("f32", 64, 64), ("bf16", 32, 64), ("bf16", 64, 32)]:
        a = args(variant="F1A", dtype=dt, dk=dk, dv=dv)
        assert _names(lib, a) == ["a_segment", "a_segscan", "a_output"], (dt, dk, dv)


def test_single_token_takes_the_decode_kernel(lib):
    """seqlen = 1 runs the one-kernel decode step for every variant and both
    forms, with no workspace."""
    for var, W in (("F1", 1), ("F2", 1), ("F3", 5), ("F1A", 1), ("F3A", 8)):
        for chunk in (0, 64):
            a = args(variant=var, window=W, seqlen=1, chunk=chunk)
            assert _names(lib, a) == ["decode"]
            assert wsize(lib, a) == 0
            assert validate(lib, a) == fb.OK


def test_falcon2a_paths(lib):
    """Falcon-2A (variant 12): the recurrent form for any head size, the
    chunk kernel for d_k in {32, 64}, no workspace on the chunk path; it
    takes no window."""
    assert validate(lib, with_ws(lib, args(variant="F2A", chunk=0, dk=16, dv=16))) == fb.OK
    for dk in (32, 64):
        a = args(variant="F2A", dk=dk, dv=128)
        assert _names(lib, a) == ["chunk_f2a"]
        assert wsize(lib, a) == 0
        assert validate(lib, a) == fb.OK
    assert validate(lib, with_ws(lib, args(variant="F2A", dk=128))) == fb.ERR_UNSUPPORTED
    assert validate(lib, args(variant="F2A", window=2)) == fb.ERR_INVALID_ARG


def test_every_kernel_name_maps_to_its_source(lib):
    """The names falcon_kernel_name reports, over every path, are the keys
    profiles and the bench use to find each kernel's source file, and every
    name appears in that source."""
    from linear_recurrent_weight_amd.build import CSRC, KERNEL_SOURCES
    cases = [args(), args(seqlen=16384, heads=12), args(seqlen=1), args(seqlen=0), args(chunk=0),
             args(dtype="f32"), args(variant="F2"), args(variant="F2A"), args(variant="F3", window=4),
             args(variant="F1A"), args(variant="F3A", window=3), args(variant="F1A", dv=32)]
    seen = set()
    for a in cases:
        seen |= set(_names(lib, a))
    assert {"f1_segmap", "f1_segscan", "decode", "chunk_f2a"} <= seen
    for nm in seen:
        assert nm in KERNEL_SOURCES, nm
        assert nm in (CSRC / KERNEL_SOURCES[nm]).read_text(), nm


# -- falcon_bwd (Falcon-1 backward) ---------------------------------------------

def bargs(**kw):
    base = dict(dtype="bf16", batch=2, heads=3, seqlen=100, dk=64, dv=64, q=FAKE, k=2 * FAKE,
                v=3 * FAKE, beta=4 * FAKE, lam=5 * FAKE, d_o=6 * FAKE, d_q=7 * FAKE, d_k=8 * FAKE,
                d_v=9 * FAKE, d_beta=10 * FAKE, d_lam=11 * FAKE)
    base.update(kw)
    return fb.make_bwd_args(**base)


def bwd_wsize(lib, a):
    return lib.falcon_bwd_workspace_size(ctypes.byref(a))


def bwd_validate(lib, a):
    return lib.falcon_bwd_validate(ctypes.byref(a))


def test_bwd_workspace_layout(lib):
    """Chunk-parallel form (T > 0, d_k and d_v at most 64): per 64-token
    chunk an fp32 record of A [d_k][d_k], B and G^T dO [d_k][d_v]; the entry
    state of every chunk plus S_T; the state gradient at every chunk's end;
    one float per chunk and 16 value columns.  Token-recurrent form (the other
    shapes): fp32 features and step scalars, the state before every 4th token
    of every head, the residuals r_t (d_v per token), and the sweep's partial
    sums (4 + 2 d_k floats per token and group of 16 value columns).  Each
    piece 256-byte aligned."""
    align = lambda n: -(-n // 256) * 256
    for B, H, T, dk, dv in [(2, 3, 100, 64, 64), (1, 1, 7, 16, 32), (4, 3, 1024, 32, 64), (2, 1, 64, 64, 16)]:
        bh, nck = B * H, -(-T // 64)
        want = (align(bh * nck * (dk * dk + 2 * dk * dv) * 4) + align(bh * (nck + 1) * dk * dv * 4)
                + align(bh * nck * dk * dv * 4) + align(bh * nck * (dv // 16) * 4))
        assert bwd_wsize(lib, bargs(batch=B, heads=H, seqlen=T, dk=dk, dv=dv)) == want
    for B, H, T, dk, dv in [(1, 1, 7, 16, 128), (3, 2, 0, 128, 16), (2, 2, 0, 64, 64), (1, 2, 90, 128, 128)]:
        bh = B * H
        want = (2 * align(bh * T * dk * 4) + 2 * align(bh * T * 4) + align(bh * -(-T // 4) * dk * dv * 4)
                + align(bh * T * dv * 4) + align(bh * T * (dv // 16) * (4 + 2 * dk) * 4))
        assert bwd_wsize(lib, bargs(batch=B, heads=H, seqlen=T, dk=dk, dv=dv)) == want


def test_bwd_rules(lib):
    a = bargs()
    n = bwd_wsize(lib, a)
    ok = bargs(workspace=1 << 40, workspace_bytes=n)
    assert bwd_validate(lib, ok) == fb.OK
    assert bwd_validate(lib, bargs()) == fb.ERR_WORKSPACE
    for var in ("F2", "F3", "F1A", "F2A", "F3A"):
        assert bwd_validate(lib, bargs(variant=var, workspace=1 << 40, workspace_bytes=n)) == fb.ERR_UNSUPPORTED
    assert bwd_validate(lib, bargs(variant=14)) == fb.ERR_INVALID_ARG
    assert bwd_validate(lib, bargs(dk=48)) == fb.ERR_UNSUPPORTED
    assert bwd_validate(lib, bargs(eps_gamma=1.0)) == fb.ERR_INVALID_ARG
    assert bwd_validate(lib, bargs(d_o=None, workspace=1 << 40, workspace_bytes=n)) == fb.ERR_INVALID_ARG
    assert bwd_validate(lib, bargs(d_q=FAKE + 8, workspace=1 << 40, workspace_bytes=n)) == fb.ERR_INVALID_ARG
    # an output on top of an input
    assert bwd_validate(lib, bargs(d_v=3 * FAKE, workspace=1 << 40, workspace_bytes=n)) == fb.ERR_INVALID_ARG
    # two outputs on top of each other
    assert bwd_validate(lib, bargs(d_k=7 * FAKE, workspace=1 << 40, workspace_bytes=n)) == fb.ERR_INVALID_ARG
    # tail pairs belong to window variants
    st = fb.FalconStateC(12 * FAKE, 13 * FAKE, 14 * FAKE, 15 * FAKE, 1, 0)
    assert bwd_validate(lib, bargs(state_in=st, workspace=1 << 40, workspace_bytes=n)) == fb.ERR_INVALID_ARG
    st = fb.FalconStateC(12 * FAKE, 13 * FAKE, None, None, 0, 0)
    assert bwd_validate(lib, bargs(state_in=st, workspace=1 << 40, workspace_bytes=n)) == fb.OK
    st = fb.FalconStateC(12 * FAKE, None, None, None, 0, 0)      # continued without x_next
    assert bwd_validate(lib, bargs(state_in=st, workspace=1 << 40, workspace_bytes=n)) == fb.ERR_INVALID_ARG


def test_bwd_kernel_names(lib):
    from linear_recurrent_weight_amd.build import CSRC, KERNEL_SOURCES

    def names(a):
        out = []
        while (nm := lib.falcon_bwd_kernel_name(ctypes.byref(a), len(out))) is not None:
            out.append(nm.decode())
        return out
    assert names(bargs()) == ["bwd_ops", "bwd_carry_fwd", "bwd_carry_rev", "bwd_grads"]
    assert names(bargs(dk=128)) == ["feature", "bwd_states", "bwd_sweep", "bwd_reduce"]
    assert names(bargs(dv=128)) == ["feature", "bwd_states", "bwd_sweep", "bwd_reduce"]
    assert names(bargs(seqlen=0)) == ["bwd_states", "bwd_sweep"]
    assert names(bargs(variant="F2")) == []
    for nm in names(bargs()) + names(bargs(dk=128)):
        assert nm in (CSRC / KERNEL_SOURCES[nm]).read_text()
