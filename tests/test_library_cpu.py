"""The C-ABI library loads, exports every symbol include/jsverify.h declares, and
rejects bad arguments on the host with the documented status codes.  No call here
reaches a kernel launch: every case fails validation first (CPU only)."""
import ctypes
import re
from pathlib import Path

import pytest

from draft_block_verification_rmsnorm_amd import jsverify as J

ROOT = Path(__file__).resolve().parents[1]
FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails before any use


def declared_functions():
    text = (ROOT / "include" / "jsverify.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jsv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return J.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("jsv_lmhead_logits", "jsv_verify_block", "jsv_score_outcomes", "jsv_workspace_bytes"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(J.EXPORTED) == set(declared_functions())


def test_status_strings_and_version(lib):
    assert lib.jsv_status_string(0) == b"ok"
    assert lib.jsv_status_string(-3) == b"workspace too small"
    assert lib.jsv_version() >= 100


def head(vocab=151936, hidden=4096, dtype=J.JSV_BF16, weight=FAKE, norm=FAKE, eps=1e-6):
    return J._Head(weight, norm, vocab, hidden, eps, dtype)


def test_workspace_bytes(lib):
    h = head()
    n16 = lib.jsv_workspace_bytes(ctypes.byref(h), 1, 16, 8)
    n32 = lib.jsv_workspace_bytes(ctypes.byref(h), 4, 32, 8)
    assert n16 >= 17 * 151936 * 4 and n32 >= 132 * 151936 * 4 and n32 > n16
    for args in [(0, 16, 8), (9, 16, 8), (1, 0, 8), (1, 33, 8), (1, 16, 65), (1, 16, -1)]:
        assert lib.jsv_workspace_bytes(ctypes.byref(h), *args) == 0
    assert lib.jsv_workspace_bytes(None, 1, 16, 8) == 0
    for bad in [head(hidden=4000), head(hidden=8192 * 2), head(dtype=7), head(vocab=0),
                head(weight=0), head(weight=FAKE + 8), head(eps=-1.0)]:
        assert lib.jsv_workspace_bytes(ctypes.byref(bad), 1, 16, 8) == 0


def test_workspace_holds_the_split_d_planes(lib):
    """34..144 rows on a bf16 head with d a multiple of 1024 (up to 5120) take the split-d
    LM head: the workspace then also holds the normalised rows and the fp32 partial-product
    planes (blocks x V x rows rounded up to 16).  Other heads and row counts do not."""
    V = 151936
    bf = head(vocab=V, hidden=4096)
    n_wide = lib.jsv_workspace_bytes(ctypes.byref(bf), 4, 32, 8)       # 132 rows
    planes = 4 * V * 144 * 4
    assert n_wide >= planes + 132 * V * 4 + 132 * 4096 * 2
    fp8 = head(vocab=V, hidden=4096, dtype=J.JSV_FP8)
    n_fp8 = lib.jsv_workspace_bytes(ctypes.byref(fp8), 4, 32, 8)
    assert n_fp8 < planes                                               # row passes, no planes
    # one pass of rows (B (K + 1) <= 33) never needs the planes
    assert lib.jsv_workspace_bytes(ctypes.byref(bf), 1, 32, 8) < planes
    # d = 3072 is three blocks, d = 5120 five
    d3 = head(vocab=V, hidden=3072)
    assert lib.jsv_workspace_bytes(ctypes.byref(d3), 2, 32, 8) >= 3 * V * 80 * 4
    d5 = head(vocab=V, hidden=5120)
    assert lib.jsv_workspace_bytes(ctypes.byref(d5), 4, 32, 8) >= 5 * V * 144 * 4
    # a workspace sized for a larger block (264 rows: row passes) also covers the smaller
    # blocks that take the split-d path
    assert lib.jsv_workspace_bytes(ctypes.byref(bf), 8, 32, 8) >= n_wide
    for b, k in [(1, 16), (2, 16), (4, 16), (4, 32), (8, 16), (8, 32)]:
        assert lib.jsv_workspace_bytes(ctypes.byref(bf), 8, 32, 8) >= lib.jsv_workspace_bytes(ctypes.byref(bf), b, k, 8)


def _verify(lib, h=None, **kw):
    a = dict(hidden=FAKE, drafts=FAKE, dl=FAKE, B=1, K=16, T=1.0, mode=0, seed=0, offset=0,
             nacc=FAKE, comm=FAKE, flags=0, lout=0, ws=FAKE, wsb=1 << 40, stream=0)
    a.update(kw)
    h = h or head()
    return lib.jsv_verify_block(ctypes.byref(h), a["hidden"], a["drafts"], a["dl"], a["B"], a["K"],
                                a["T"], a["mode"], a["seed"], a["offset"], a["nacc"], a["comm"],
                                a["flags"], a["lout"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), J.JSV_EINVAL), (dict(B=9), J.JSV_EINVAL), (dict(K=0), J.JSV_EINVAL),
    (dict(K=33), J.JSV_EINVAL), (dict(T=-1.0), J.JSV_EINVAL), (dict(T=float("nan")), J.JSV_EINVAL),
    (dict(T=float("inf")), J.JSV_EINVAL), (dict(mode=2), J.JSV_EINVAL),
    (dict(hidden=0), J.JSV_EINVAL), (dict(hidden=FAKE + 4), J.JSV_EINVAL),
    (dict(drafts=0), J.JSV_EINVAL), (dict(nacc=0), J.JSV_EINVAL), (dict(comm=0), J.JSV_EINVAL),
    (dict(ws=0), J.JSV_EINVAL), (dict(dl=0), J.JSV_EINVAL),            # softmax at T > 0 needs q
    (dict(wsb=1000), J.JSV_EWORKSPACE),
])
def test_verify_argument_errors(lib, kw, code):
    assert _verify(lib, **kw) == code


def test_verify_shape_errors(lib):
    assert _verify(lib, h=head(hidden=4000)) == J.JSV_EUNSUPPORTED
    assert _verify(lib, h=head(hidden=256 * 64)) == J.JSV_EUNSUPPORTED
    assert _verify(lib, h=head(dtype=3)) == J.JSV_EINVAL
    assert _verify(lib, h=head(vocab=-5)) == J.JSV_EINVAL
    assert _verify(lib, h=head(vocab=2 ** 31)) == J.JSV_EUNSUPPORTED
    # the workspace check counts the logits only when the caller gives no logits_out
    h = head()
    need = lib.jsv_workspace_bytes(ctypes.byref(h), 1, 16, 0)
    assert _verify(lib, wsb=need - 1) == J.JSV_EWORKSPACE


def test_score_argument_errors(lib):
    h = head()

    def call(top_n=8, hidden=FAKE, out=FAKE, T=1.0, dl=FAKE, wsb=1 << 40):
        return lib.jsv_score_outcomes(ctypes.byref(h), hidden, FAKE, dl, 1, 16, T, 0, top_n,
                                      out, out, out, 0, 0, FAKE, wsb, 0)

    assert call(top_n=0) == J.JSV_EINVAL
    assert call(top_n=65) == J.JSV_EINVAL
    assert call(hidden=0) == J.JSV_EINVAL
    assert call(out=0) == J.JSV_EINVAL
    assert call(dl=0) == J.JSV_EINVAL
    assert call(wsb=10) == J.JSV_EWORKSPACE


def test_lmhead_argument_errors(lib):
    h = head()
    assert lib.jsv_lmhead_logits(ctypes.byref(h), FAKE, -1, FAKE, 0, 0, 0) == J.JSV_EINVAL
    assert lib.jsv_lmhead_logits(ctypes.byref(h), FAKE, 0, FAKE, 0, 0, 0) == J.JSV_OK  # empty input
    assert lib.jsv_lmhead_logits(ctypes.byref(h), 0, 4, FAKE, 0, 0, 0) == J.JSV_EINVAL
    assert lib.jsv_lmhead_logits(ctypes.byref(h), FAKE, 4, 0, 0, 0, 0) == J.JSV_EINVAL
    bad = head(hidden=100)
    assert lib.jsv_lmhead_logits(ctypes.byref(bad), FAKE, 4, FAKE, 0, 0, 0) == J.JSV_EUNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        J.load_library(tmp_path / "libjsverify.so")


def test_next_row_argument_errors(lib):
    h = head()
    st = lib.jsv_anchor_replace(ctypes.byref(h), FAKE, FAKE, 0, 16, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == J.JSV_EINVAL
    st = lib.jsv_anchor_replace(ctypes.byref(h), FAKE, FAKE, 1, 16, None, FAKE, None, FAKE, 1 << 40, None)
    assert st == J.JSV_EINVAL
    st = lib.jsv_anchor_replace(ctypes.byref(h), FAKE, FAKE, 1, 16, FAKE, FAKE, None, FAKE, 10, None)
    assert st == J.JSV_EWORKSPACE
    assert lib.jsv_cache_lookup(FAKE, FAKE, 1, 16, FAKE, FAKE, 0, FAKE, None) == J.JSV_EINVAL
    assert lib.jsv_cache_lookup(FAKE, FAKE, 1, 33, FAKE, FAKE, 8, FAKE, None) == J.JSV_EINVAL
    assert lib.jsv_cache_lookup(None, FAKE, 1, 16, FAKE, FAKE, 8, FAKE, None) == J.JSV_EINVAL
    assert lib.jsv_calibrated_lengths(FAKE, 1, 0, FAKE, None, None) == J.JSV_EINVAL
    assert lib.jsv_calibrated_lengths(None, 1, 4, FAKE, None, None) == J.JSV_EINVAL


def test_geometric_fanout_matches_oracle():
    """The host fan-out is plain C in the library (no device work), so its parity with
    the oracle is checked here, on the CPU."""
    import numpy as np
    import oracle
    for alpha, rho, gamma, B in [(0.6, 1.0, 4, 10), (0.8, 0.5, 15, 16), (0.3, 2.0, 3, 6),
                                 (0.93, 1.2, 31, 16), (0.5, 1.0, 6, 4), (0.99, 0.3, 64, 1000)]:
        fr, fi, hm = J.geometric_fanout(alpha, rho, gamma, B)
        F, Fi, obj, _ = oracle.geometric_fanout(alpha, rho, gamma, B)
        assert np.allclose(fr, F, rtol=1e-12, atol=1e-12), (alpha, rho, gamma, B)
        assert list(fi) == [int(x) for x in Fi], (alpha, rho, gamma, B)
        assert abs(hm - obj) < 1e-12
    fr, fi, hm = J.geometric_fanout(0.6, 1.0, 4, 10)
    assert abs(hm - 0.567) < 5e-4 and fi == [3, 3, 2, 0, 2]
    for bad in [(0.0, 1.0, 4, 10), (1.0, 1.0, 4, 10), (0.5, 0.0, 4, 10), (0.5, 1.0, 4, 1)]:
        with pytest.raises(RuntimeError):
            J.geometric_fanout(*bad)
    with pytest.raises(ValueError):
        J.geometric_fanout(0.5, 1.0, 0, 10)


def test_fp8_head_validation(lib):
    ok = J._Head(FAKE, FAKE, 151936, 4096, 1e-6, J.JSV_FP8, FAKE)
    assert lib.jsv_workspace_bytes(ctypes.byref(ok), 1, 16, 8) > 0
    no_scale = J._Head(FAKE, FAKE, 151936, 4096, 1e-6, J.JSV_FP8, None)
    assert lib.jsv_workspace_bytes(ctypes.byref(no_scale), 1, 16, 8) == 0
    odd_steps = J._Head(FAKE, FAKE, 1024, 256, 1e-6, J.JSV_FP8, FAKE)   # one k-step per wave
    assert lib.jsv_workspace_bytes(ctypes.byref(odd_steps), 1, 16, 8) == 0
