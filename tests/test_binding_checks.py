"""The Python binding rejects tensors that do not match the shapes, dtypes,
devices and layouts the C ABI assumes, before anything reaches the library
(the library sees only pointers and sizes).  CPU only: the checks run on
host tensors."""
from __future__ import annotations

import pytest

torch = pytest.importorskip("torch")

from linear_recurrent_weight_amd import falcon as fb


def tensors(B=2, H=3, T=10, dk=16, dv=8, dtype=torch.float32, variant="F1"):
    q = torch.zeros(B, H, T, dk, dtype=dtype)
    k = torch.zeros(B, H, T, dk, dtype=dtype)
    v = torch.zeros(B, H, T, dv, dtype=dtype)
    beta = torch.zeros(B, H, T, dv) if variant == "F2" else torch.zeros(B, H, T)
    lam = torch.zeros(B, H, T)
    return q, k, v, beta, lam


def check(*t, **kw):
    kw.setdefault("variant", "F1")
    kw.setdefault("window", 1)
    return fb.check_fwd_tensors(*t, **kw)


def test_matching_tensors_pass():
    assert check(*tensors())[:5] == (2, 3, 10, 16, 8)
    assert check(*tensors(variant="F2"), variant="F2")[4] == 8
    st = fb.FalconState.empty(2, 3, 16, 8, 4, "cpu")
    st.n_tail, st.fresh = 2, False
    check(*tensors(), variant="F3A", window=4, state=st, out=torch.zeros(2, 3, 10, 8))


@pytest.mark.parametrize("which,bad", [
    ("k", torch.zeros(2, 3, 10, 32)),               # k vs q head dim
    ("k", torch.zeros(2, 3, 11, 16)),               # length
    ("v", torch.zeros(2, 2, 10, 8)),                # heads
    ("beta", torch.zeros(2, 3, 10, 8)),             # a per-column gain for Falcon-1
    ("lam", torch.zeros(2, 3, 9)),
    ("beta", torch.zeros(2, 3, 10, dtype=torch.float64)),
    ("k", torch.zeros(2, 3, 10, 16, dtype=torch.bfloat16)),   # mixed io dtypes
    ("v", torch.zeros(2, 3, 8, 10).transpose(2, 3)),          # not contiguous
    ("lam", torch.zeros(2, 3, 10, device="meta")),            # another device
])
def test_mismatched_input_is_rejected(which, bad):
    t = dict(zip(("q", "k", "v", "beta", "lam"), tensors()))
    t[which] = bad
    with pytest.raises(ValueError):
        check(t["q"], t["k"], t["v"], t["beta"], t["lam"])


def test_falcon2_needs_per_column_gains():
    with pytest.raises(ValueError):
        check(*tensors(), variant="F2")


def test_output_must_match():
    with pytest.raises(ValueError):
        check(*tensors(), out=torch.zeros(2, 3, 10, 16))
    with pytest.raises(ValueError):
        check(*tensors(), out=torch.zeros(2, 3, 10, 8, dtype=torch.bfloat16))


def test_state_must_match():
    st = fb.FalconState.empty(2, 3, 16, 16, 1, "cpu")       # S with d_v = 16, not 8
    with pytest.raises(ValueError):
        check(*tensors(), state=st)
    st = fb.FalconState.empty(2, 3, 16, 8, 1, "cpu")
    st.fresh = False
    st.x_next = torch.zeros(2, 3, 8)                        # x_next needs d_k entries
    with pytest.raises(ValueError):
        check(*tensors(), state=st)


def test_tail_from_a_narrower_window_is_rejected():
    """A state carried out of a W = 3 call holds two tail slots; a W = 8 call
    would index seven."""
    st = fb.FalconState.empty(2, 3, 16, 8, 3, "cpu")
    st.n_tail, st.fresh = 2, False
    check(*tensors(), variant="F3A", window=3, state=st)
    with pytest.raises(ValueError):
        check(*tensors(), variant="F3A", window=8, state=st)


def test_tail_count_bounds():
    st = fb.FalconState.empty(2, 3, 16, 8, 3, "cpu")
    st.n_tail, st.fresh = 3, False
    with pytest.raises(ValueError):
        check(*tensors(), variant="F3A", window=3, state=st)
    st.n_tail, st.fresh = 1, True
    with pytest.raises(ValueError):
        check(*tensors(), variant="F3A", window=3, state=st)


def test_fwd_refuses_host_tensors():
    if not fb.LIB_PATH.exists():
        pytest.skip("libfalcon.so not built")
    with pytest.raises(ValueError):
        fb.fwd(*tensors())
