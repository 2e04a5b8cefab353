"""Bank files (CPU): save / load round trips, the header, and every failure the loader
must detect (a flipped byte in any section, truncation, a foreign file, a bank of another
shape, offsets that break the chunking rule)."""
import os

import numpy as np
import pytest
import torch

M = pytest.importorskip("latent_memory_long_amd")
from latent_memory_long_amd.binding import MsaError  # noqa: E402

IO, INVALID = 5, 1


def _kr_elems(dtype, C, h_r=3, d=32):
    return M.msa_krbar_elems(0 if dtype == torch.float32 else 1, C, h_r, d)


def _bank(seed, n_docs=23, layers=2, dtype=torch.bfloat16, h_kv=2, h_r=3, d=32, chunk=64):
    """Random bank contents (the files store bytes; routing keys as RouteKeys storage of the
    bank layout's size: 16-row tiles for bf16)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 300, size=n_docs)
    dto = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    cho = M.msa_chunk_offsets(dto, chunk)
    C = int(cho[-1])
    g = torch.Generator().manual_seed(seed)
    keys = lambda: M.RouteKeys(torch.randn(_kr_elems(dtype, C, h_r, d), generator=g).to(dtype), C, h_r, d)
    trio = lambda: (keys(), torch.randn((C, h_kv, d), generator=g).to(dtype), torch.randn((C, h_kv, d), generator=g).to(dtype))
    return dto, cho, [trio() for _ in range(layers)]


def _same(x, y):
    if isinstance(x, M.RouteKeys):
        return x.shape == y.shape and _same(x.data, y.data)
    return x.dtype == y.dtype and torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                                              y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


@pytest.mark.parametrize("dtype,layers", [(torch.bfloat16, 1), (torch.bfloat16, 3), (torch.float32, 2)])
def test_round_trip(tmp_path, dtype, layers):
    dto, cho, L = _bank(1, layers=layers, dtype=dtype)
    path = str(tmp_path / "bank.msab")
    M.msa_bank_save(path, dto, cho, L, chunk=64, rope_base=1e6, rope_mask=M.MSA_ROPE_K)
    info = M.msa_bank_read_info(path)
    assert info["n_layers"] == layers and info["n_docs"] == len(dto) - 1 and info["n_chunks"] == cho[-1]
    assert info["n_tokens"] == dto[-1] and info["chunk"] == 64 and info["rope_base"] == 1e6
    assert info["rope_mask"] == M.MSA_ROPE_K and info["dtype"] == (0 if dtype == torch.float32 else 1)
    d2, c2, L2, _ = M.msa_bank_load(path)
    assert np.array_equal(d2, dto) and np.array_equal(c2, cho)
    for a, b in zip(L, L2):
        for x, y in zip(a, b):
            assert _same(x, y)
    # the file size is exactly header + sections + checksums + end mark; bf16 routing keys
    # fill whole 16-row tiles
    esz = 4 if dtype == torch.float32 else 2
    C, n = int(cho[-1]), len(dto)
    kr = _kr_elems(dtype, C)
    assert kr == (C if dtype == torch.float32 else (C + 15) // 16 * 16) * 3 * 32
    expect = 8 + 64 + 2 * n * 8 + layers * (kr + C * (2 + 2) * 32) * esz + (2 + 3 * layers) * 8 + 8
    assert os.path.getsize(path) == expect


def _expect_error(path, code, text):
    with pytest.raises(MsaError) as e:
        M.msa_bank_load(path)
    assert e.value.status == code and text in str(e.value), str(e.value)


def test_every_section_is_checked(tmp_path):
    dto, cho, L = _bank(2, layers=2)
    path = str(tmp_path / "bank.msab")
    M.msa_bank_save(path, dto, cho, L)
    blob = bytearray(open(path, "rb").read())
    n, C = len(dto), int(cho[-1])
    starts = [72, 72 + n * 8]                       # the two offset arrays
    pos = 72 + 2 * n * 8
    for _ in range(2):
        for n_el in (_kr_elems(torch.bfloat16, C), C * 2 * 32, C * 2 * 32):   # Kr-bar, K-bar, V-bar
            starts.append(pos)
            pos += n_el * 2
    names = ["doc_tok_off", "chunk_off"] + [f"layer {l} {t}" for l in range(2) for t in ("Kr-bar", "K-bar", "V-bar")]
    for start, name in zip(starts, names):
        bad = bytearray(blob)
        bad[start + 3] ^= 0x40
        p = str(tmp_path / "bad.msab")
        open(p, "wb").write(bytes(bad))
        _expect_error(p, IO, "checksum mismatch in " + name)


def test_truncated_foreign_and_mismatched_files(tmp_path):
    dto, cho, L = _bank(3)
    path = str(tmp_path / "bank.msab")
    M.msa_bank_save(path, dto, cho, L)
    blob = open(path, "rb").read()
    p = str(tmp_path / "short.msab")
    open(p, "wb").write(blob[:-20])
    _expect_error(p, IO, "truncated")
    open(p, "wb").write(blob + b"x")
    _expect_error(p, IO, "malformed")
    open(p, "wb").write(b"not a bank file at all" * 4)
    _expect_error(p, IO, "not a bank file")
    _expect_error(str(tmp_path / "missing.msab"), IO, "cannot open")
    # buffers sized for another bank are refused before anything is read into them
    info = M.binding.BankInfo()
    assert M.binding.lib.msa_bank_read_info(path.encode(), info) == 0
    info.n_chunks += 1
    null = (M.binding.ctypes.c_void_p * 1)(None)
    dummy = np.zeros(len(dto), dtype=np.int64)
    st = M.binding.lib.msa_bank_load(path.encode(), info, dummy.ctypes.data, dummy.ctypes.data, null, null, null)
    assert st == INVALID and "differs" in M.msa_last_error()


def test_save_rejects_offsets_that_break_the_chunking_rule(tmp_path):
    dto, cho, L = _bank(4)
    bad = cho.copy()
    bad[5] += 1                                      # document 4 claims a row of document 5
    with pytest.raises(MsaError) as e:
        M.msa_bank_save(str(tmp_path / "b.msab"), dto, bad, L)
    assert e.value.status == INVALID and "rows for" in str(e.value)
    assert not os.path.exists(tmp_path / "b.msab")
