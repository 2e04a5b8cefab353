"""Host-side tests of the C ABI (no GPU needed): the library loads, exports every entry
point declared in include/msa.h, computes the bank layout on the host, and rejects bad
arguments with the documented status codes before making any HIP call."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import msa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

m = pytest.importorskip("latent_memory_long_amd")
lib = m.binding.lib
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (msa_\w+)", out))
    assert set(names) <= exported, set(names) - exported


def test_library_targets_gfx950():
    blob = open(m.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_status_strings_and_version():
    assert m.msa_version() >= 10000
    assert m.msa_status_string(0) == "ok"
    assert "workspace" in m.msa_status_string(3)


def test_chunk_offsets_match_oracle():
    rng = np.random.default_rng(0)
    for chunk in (1, 7, 64, 128):
        lens = rng.integers(1, 500, size=rng.integers(1, 60))
        off = np.concatenate([[0], np.cumsum(lens)])
        got = m.msa_chunk_offsets(off, chunk)
        assert np.array_equal(got, O.chunk_offsets(lens, chunk))
    assert list(m.msa_chunk_offsets([0, 180], 64)) == [0, 3]


@pytest.mark.parametrize("off,chunk", [([0, 5, 5], 64), ([1, 5], 64), ([0, 5], 0)])
def test_chunk_offsets_rejects(off, chunk):
    with pytest.raises(m.MsaError):
        m.msa_chunk_offsets(off, chunk)


def _pool(**kw):
    a = dict(dtype=1, n_docs=2, n_tokens=10, n_chunks=2, off=FAKE, coff=FAKE, h_kv=8, h_r=8, d=128,
             chunk=64, base=1e6, mask=1, K=FAKE, V=FAKE, Kr=FAKE, Kb=FAKE, Vb=FAKE, Krb=FAKE)
    a.update(kw)
    return lib.msa_pool(a["dtype"], a["n_docs"], a["n_tokens"], a["n_chunks"], a["off"], a["coff"],
                        a["h_kv"], a["h_r"], a["d"], a["chunk"], a["base"], a["mask"], a["K"], a["V"],
                        a["Kr"], a["Kb"], a["Vb"], a["Krb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), UNSUPPORTED), (dict(n_docs=0), INVALID), (dict(n_tokens=1), INVALID),
    (dict(n_chunks=11), INVALID), (dict(K=None), INVALID), (dict(coff=None), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(h_kv=0), UNSUPPORTED), (dict(chunk=0), UNSUPPORTED),
    (dict(chunk=129), UNSUPPORTED), (dict(mask=8), INVALID), (dict(base=-1.0), INVALID),
])
def test_pool_validation(kw, code):
    assert _pool(**kw) == code
    assert lib.msa_last_error().decode()


def _route(**kw):
    a = dict(dtype=1, B=1, total_q=64, q_off=FAKE, maxq=64, Qr=FAKE, h_r=8, d=128, N=10, C=20,
             coff=FAKE, Krb=FAKE, k=4, ids=FAKE, sc=FAKE, ds=None, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return lib.msa_route_topk(a["dtype"], a["B"], a["total_q"], a["q_off"], a["maxq"], a["Qr"],
                              a["h_r"], a["d"], a["N"], a["C"], a["coff"], a["Krb"], a["k"], a["ids"],
                              a["sc"], a["ds"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), UNSUPPORTED), (dict(B=0), INVALID), (dict(maxq=0), INVALID),
    (dict(Qr=None), INVALID), (dict(h_r=17), UNSUPPORTED), (dict(d=96), UNSUPPORTED),
    (dict(N=0), INVALID), (dict(C=5), INVALID), (dict(k=0), INVALID), (dict(k=1025), UNSUPPORTED),
    (dict(ids=None), INVALID), (dict(wsb=16), WORKSPACE), (dict(ws=None), WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x1010)), INVALID),
])
def test_route_validation(kw, code):
    assert _route(**kw) == code
    assert lib.msa_last_error().decode()


def _attn(**kw):
    a = dict(dtype=1, B=1, tq=64, tkv=64, q_off=FAKE, kv_off=FAKE, maxq=64, Q=FAKE, Kl=FAKE, Vl=FAKE,
             hq=32, h_kv=8, d=128, base=1e6, scale=0.0, k=16, ids=FAKE, N=10, C=20, coff=FAKE,
             Kb=FAKE, Vb=FAKE, src=0, O=FAKE, lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.msa_sparse_attn(a["dtype"], a["B"], a["tq"], a["tkv"], a["q_off"], a["kv_off"], a["maxq"],
                               a["Q"], a["Kl"], a["Vl"], a["hq"], a["h_kv"], a["d"], a["base"], a["scale"],
                               a["k"], a["ids"], a["N"], a["C"], a["coff"], a["Kb"], a["Vb"], a["src"],
                               a["O"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), UNSUPPORTED), (dict(tkv=10), INVALID), (dict(hq=30), INVALID),
    (dict(d=100), UNSUPPORTED), (dict(k=0), INVALID), (dict(k=2048), UNSUPPORTED),
    (dict(src=2), INVALID), (dict(wsb=100), WORKSPACE), (dict(base=0.0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(Q=None), INVALID), (dict(ids=None), INVALID),
    (dict(C=3), INVALID),
])
def test_attn_validation(kw, code):
    assert _attn(**kw) == code
    assert lib.msa_last_error().decode()


def _attn_bwd(**kw):
    a = dict(dtype=1, B=1, tq=64, tkv=64, q_off=FAKE, kv_off=FAKE, maxq=64, Q=FAKE, Kl=FAKE, Vl=FAKE,
             hq=32, h_kv=8, d=128, base=1e6, scale=0.0, k=16, ids=FAKE, N=10, C=20, coff=FAKE,
             Kb=FAKE, Vb=FAKE, src=0, O=FAKE, lse=None, dO=FAKE, dQ=FAKE, dKl=FAKE, dVl=FAKE, dKb=FAKE,
             dVb=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.msa_sparse_attn_backward(
        a["dtype"], a["B"], a["tq"], a["tkv"], a["q_off"], a["kv_off"], a["maxq"], a["Q"], a["Kl"], a["Vl"],
        a["hq"], a["h_kv"], a["d"], a["base"], a["scale"], a["k"], a["ids"], a["N"], a["C"], a["coff"],
        a["Kb"], a["Vb"], a["src"], a["O"], a["lse"], a["dO"], a["dQ"], a["dKl"], a["dVl"], a["dKb"], a["dVb"],
        a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(tkv=10), INVALID),
    (dict(hq=30), INVALID), (dict(k=2048), UNSUPPORTED), (dict(src=2), INVALID),
    (dict(wsb=100), WORKSPACE), (dict(dO=None), INVALID), (dict(dKb=None), INVALID),
    (dict(dKl=None), INVALID), (dict(O=None), INVALID), (dict(C=3), INVALID),
])
def test_attn_backward_validation(kw, code):
    assert _attn_bwd(**kw) == code
    assert lib.msa_last_error().decode()


def _route_bwd(**kw):
    a = dict(dtype=1, B=2, tq=8, q_off=FAKE, maxq=4, Qr=FAKE, h_r=4, d=128, N=10, C=20, coff=FAKE,
             Krb=FAKE, dD=FAKE, rs=None, ra=None, dQr=FAKE, dKrb=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.msa_route_backward(a["dtype"], a["B"], a["tq"], a["q_off"], a["maxq"], a["Qr"], a["h_r"], a["d"],
                                  a["N"], a["C"], a["coff"], a["Krb"], a["dD"], a["rs"], a["ra"], a["dQr"],
                                  a["dKrb"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), UNSUPPORTED), (dict(h_r=17), UNSUPPORTED), (dict(d=100), UNSUPPORTED),
    (dict(C=3), INVALID), (dict(B=0), INVALID), (dict(maxq=0), INVALID), (dict(dD=None), INVALID),
    (dict(dKrb=None), INVALID), (dict(dQr=None), INVALID), (dict(wsb=100), WORKSPACE),
    (dict(ws=None), WORKSPACE), (dict(ws=ctypes.c_void_p(0x1010)), INVALID), (dict(rs=FAKE), INVALID),
    (dict(ra=FAKE), INVALID),
])
def test_route_backward_validation(kw, code):
    assert _route_bwd(**kw) == code
    assert lib.msa_last_error().decode()


def _aux(**kw):
    a = dict(kind=0, B=2, N=10, S=FAKE, Y=FAKE, tau=1.0, loss=FAKE, dD=FAKE)
    a.update(kw)
    return lib.msa_route_aux_loss(a["kind"], a["B"], a["N"], a["S"], a["Y"], a["tau"], a["loss"], a["dD"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kind=2), UNSUPPORTED), (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(tau=0.0), INVALID),
    (dict(tau=float("inf")), INVALID), (dict(S=None), INVALID), (dict(Y=None), INVALID),
    (dict(loss=None), INVALID), (dict(dD=None), INVALID),
])
def test_aux_loss_validation(kw, code):
    assert _aux(**kw) == code
    assert lib.msa_last_error().decode()


def test_workspace_sizes():
    assert m.msa_route_topk_workspace(1, 47000, 16) >= 47000 * 4
    assert m.msa_route_topk_workspace(0, 10, 1) == 0
    a = m.msa_sparse_attn_workspace(1, 1, 64, 64, 64, 32, 8, 128)
    assert a >= 64 * 32 * 128 * 2 + 64 * 8 * 128 * 2
    assert m.msa_sparse_attn_workspace(1, 1, 64, 64, 64, 30, 8, 128) == 0
    b = m.msa_sparse_attn_backward_workspace(64, 64, 32, 8, 128)
    # rotated Q and local K, the cos / sin table of up to 1024 + total_kv positions, two floats per row
    assert b >= 64 * 32 * 128 * 2 + 64 * 8 * 128 * 2 + (1024 + 64) * 128 * 4 + 2 * 64 * 32 * 4
    assert m.msa_sparse_attn_backward_workspace(64, 64, 32, 8, 32) == 0
    c = m.msa_route_backward_workspace(2, 10, 20, 4)
    assert c >= 2 * 10 * 4 + 2 * 2 * 20 * 4 + 2 * 10 * (4 + 8) + 2 * 2 * 10 * 4 * 4
    assert m.msa_route_backward_workspace(2, 10, 5, 4) == 0 and m.msa_route_backward_workspace(2, 10, 20, 17) == 0


def test_route_scan_rows_go_together():
    # row scores without row args (or the reverse) is refused before anything runs
    for rs, ra in ((FAKE, None), (None, FAKE)):
        assert lib.msa_route_scan(1, 2, 8, FAKE, 4, FAKE, 4, 128, 10, 20, FAKE, FAKE, FAKE, rs, ra, None) == INVALID
        assert "together" in lib.msa_last_error().decode()
