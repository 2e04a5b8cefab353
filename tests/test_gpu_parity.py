"""GPU parity of the HIP path against the CPU oracle, at sizes the oracle finishes in
seconds that still span many tiles and ragged tails.  Every case prints its name before
touching the GPU."""
import os

import numpy as np
import pytest
import torch

import latent_memory_long_amd as M
from oracle import msa_oracle as O
from synth import workloads as W
from tests.helpers import (as_keys, assert_attn_close, assert_pool_close, assert_scores_close,
                           assert_topk_consistent, assert_topk_valid, f64, key_rows, oracle_doc_scores_all,
                           pool_error_bound, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dt(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def _cpu_randn(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32) * std


def _route_env(path):
    if path == "auto":
        os.environ.pop("MSA_ROUTE_PATH", None)
    else:
        os.environ["MSA_ROUTE_PATH"] = path


@pytest.fixture(autouse=True)
def _reset_env():
    yield
    os.environ.pop("MSA_ROUTE_PATH", None)


def random_bank(n_chunks_per_doc, heads, d, dtype, seed, doc_std=0.5):
    """Pooled-looking bank: per-document offset plus noise, rows of each document
    contiguous.  Returns (chunk_off host, row-major tensor [C, heads, d] on the GPU); routing
    calls take it through as_keys (the library's bank layout)."""
    counts = np.asarray(n_chunks_per_doc, dtype=np.int64)
    coff = np.concatenate([[0], np.cumsum(counts)])
    mu = _cpu_randn((len(counts), heads, d), seed, doc_std)
    x = _cpu_randn((int(coff[-1]), heads, d), seed + 1, 0.125)
    x += torch.repeat_interleave(mu, torch.as_tensor(counts), dim=0)
    return coff, x.to(_dt(dtype)).to(DEV)


def route(Qr, q_lens, Krb, coff, k, want=True):
    q_off = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32, device=DEV)
    coff_d = torch.tensor(coff, dtype=torch.int64, device=DEV)
    ids, sc, ds = M.msa_route_topk(Qr, q_off, int(max(q_lens)), as_keys(Krb), coff_d, k, want_doc_scores=want)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy(), (ds.cpu().numpy() if ds is not None else None)


# ------------------------------------------------------------------------------ end to end

def test_tiny_fp32_end_to_end():
    say("case tiny_fp32 end-to-end")
    wl = W.workload("tiny_fp32")
    sh = wl.shape
    lens = W.doc_lengths(wl)
    off = W.token_offsets(lens)
    K, V, Kr = W.gen_token_states(wl, lens, "cpu")
    coff = M.msa_chunk_offsets(off, sh.chunk)
    C = int(coff[-1])
    off_d = torch.tensor(off, device=DEV)
    coff_d = torch.tensor(coff, device=DEV)
    Kb, Vb, Krb = M.msa_pool(K.to(DEV), V.to(DEV), Kr.to(DEV), off_d, coff_d, C, sh.chunk, sh.rope_base)
    oK, oV, oKr, ocoff = O.pool(f64(K), f64(V), f64(Kr), off, sh.chunk, sh.rope_base, O.ROPE_K)
    assert np.array_equal(ocoff, coff)
    for g, o, x, rot, n in ((Kb, oK, K, True, "Kbar"), (Vb, oV, V, False, "Vbar"), (Krb, oKr, Kr, False, "Krbar")):
        assert_pool_close(g, o, "f32", n, pool_error_bound(f64(x), off, sh.chunk, rot))

    q = W.gen_queries(wl, "cpu")
    Lq = int(q["q_len"][0])
    ids, sc, ds = route(q["Qr"].to(DEV), q["q_len"], Krb, coff, wl.k)
    o_ds = O.route_doc_scores(f64(q["Qr"]), [0, Lq], f64(Krb), coff)[0]
    assert_scores_close(ds[0], o_ds, "f32", "doc scores (gpu bank)")
    assert_topk_consistent(ids[0], sc[0], ds[0], wl.k, "topk")
    assert_topk_valid(ids[0], o_ds, wl.k, "topk vs oracle (gpu bank)")
    # end to end: oracle bank, oracle route
    e2e = O.route_doc_scores(f64(q["Qr"]), [0, Lq], oKr, coff)[0]
    assert_topk_valid(ids[0], e2e, wl.k, "topk vs oracle (oracle bank)")

    q_off = torch.tensor([0, Lq], dtype=torch.int32, device=DEV)
    kv_off = torch.tensor([0, int(q["kv_len"][0])], dtype=torch.int32, device=DEV)
    ids_d = torch.tensor(ids, device=DEV)
    Out = M.msa_sparse_attn(q["Q"].to(DEV), q["Kloc"].to(DEV), q["Vloc"].to(DEV), q_off, kv_off, Lq,
                            ids_d, coff_d, Kb, Vb, rope_base=sh.rope_base)
    torch.cuda.synchronize()
    ref = O.sparse_attn(f64(q["Q"]), f64(q["Kloc"]), f64(q["Vloc"]), [0, Lq], [0, int(q["kv_len"][0])],
                        ids, coff, f64(Kb), f64(Vb), sh.rope_base)
    assert_attn_close(Out, ref, "f32", "attention (gpu bank, gpu ids)")
    ref2 = O.sparse_attn(f64(q["Q"]), f64(q["Kloc"]), f64(q["Vloc"]), [0, Lq], [0, int(q["kv_len"][0])],
                         ids, coff, oK, oV, sh.rope_base)
    assert_attn_close(Out, ref2, "f32", "attention (oracle bank)")


# ------------------------------------------------------------------------------ pooling

POOL_CASES = [
    # (name, heads kv, heads r, d, chunk, rope mask, dtype)
    ("qwen_like", 8, 8, 128, 64, 1, "bf16"),
    ("rope_all", 8, 8, 128, 64, 7, "bf16"),
    ("no_rope", 8, 8, 128, 64, 0, "bf16"),
    ("d64_chunk48", 4, 2, 64, 48, 1, "bf16"),
    ("d32_chunk128", 2, 3, 32, 128, 5, "bf16"),
    ("f32_d128", 2, 2, 128, 64, 1, "f32"),
]


@pytest.mark.parametrize("case", POOL_CASES, ids=[c[0] for c in POOL_CASES])
def test_pool(case):
    name, hkv, hr, d, chunk, mask, dtype = case
    say(f"case pool {name}")
    rng = np.random.default_rng(7)
    lens = np.concatenate([[1, 63, 64, 65, 128, 129, chunk - 1, chunk + 1, 2 * chunk],
                           rng.integers(1, 700, size=25)]).astype(np.int64)
    lens = np.maximum(lens, 1)
    off = W.token_offsets(lens)
    T = int(off[-1])
    K = _cpu_randn((T, hkv, d), 1).to(_dt(dtype))
    V = _cpu_randn((T, hkv, d), 2).to(_dt(dtype))
    Kr = _cpu_randn((T, hr, d), 3).to(_dt(dtype))
    coff = M.msa_chunk_offsets(off, chunk)
    C = int(coff[-1])
    Kb, Vb, Krb = M.msa_pool(K.to(DEV), V.to(DEV), Kr.to(DEV), torch.tensor(off, device=DEV),
                             torch.tensor(coff, device=DEV), C, chunk, 1e6, mask)
    torch.cuda.synchronize()
    oK, oV, oKr, _ = O.pool(f64(K), f64(V), f64(Kr), off, chunk, 1e6, mask)
    for g, o, x, bit, n in ((Kb, oK, K, 1, "Kbar"), (Vb, oV, V, 2, "Vbar"), (Krb, oKr, Kr, 4, "Krbar")):
        r = assert_pool_close(g, o, dtype, f"{name} {n}", pool_error_bound(f64(x), off, chunk, bool(mask & bit)))
        say(f"  {name} {n}: largest error {r:.3f} of the bound")


def test_pool_constant_chunk_bit_exact_and_doc_restart():
    say("case pool constant chunk / document restart")
    d, h = 128, 8
    v = _cpu_randn((1, h, d), 11).to(torch.bfloat16)
    lens = np.array([64, 100, 1, 64], dtype=np.int64)
    K = v.repeat(int(lens.sum()), 1, 1)
    # document 3 repeats document 0's random content: identical pooled rows expected
    rnd = _cpu_randn((64, h, d), 12).to(torch.bfloat16)
    K[165:229] = rnd
    K[0:64] = rnd
    off = W.token_offsets(lens)
    coff = M.msa_chunk_offsets(off, 64)
    Kb, Vb, Krb = M.msa_pool(K.to(DEV), K.to(DEV), K.to(DEV), torch.tensor(off, device=DEV),
                             torch.tensor(coff, device=DEV), int(coff[-1]), 64, 1e6, 1)
    torch.cuda.synchronize()
    Vb, Kb, Krb = Vb.cpu(), Kb.cpu(), Krb.rows().cpu()
    # constant chunks (rows 1, 2 of document 1 and document 2) pool to the value itself
    for r in (1, 2, 3):
        assert torch.equal(Vb[r], v[0]) and torch.equal(Krb[r], v[0])
    assert torch.equal(Kb[3], v[0])          # single-token document: rotation at 0
    assert torch.equal(Kb[0], Kb[4]) and torch.equal(Vb[0], Vb[4])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pool_append_equals_pool_at_once(dtype):
    # A bank grown by appending documents (msa_pool on the new documents with offsets that
    # start after the existing rows) holds the same bits as the bank pooled in one call, and
    # routes the same.
    say(f"case pool append {dtype}")
    rng = np.random.default_rng(21)
    lens = rng.integers(1, 900, size=60).astype(np.int64)
    cut = 23
    off = W.token_offsets(lens)
    T = int(off[-1])
    h, d = 8, 128
    K = _cpu_randn((T, h, d), 31).to(_dt(dtype)).to(DEV)
    V = _cpu_randn((T, h, d), 32).to(_dt(dtype)).to(DEV)
    Kr = _cpu_randn((T, h, d), 33, 1.0).to(_dt(dtype)).to(DEV)
    coff = M.msa_chunk_offsets(off, 64)
    C = int(coff[-1])
    whole = M.msa_pool(K, V, Kr, torch.tensor(off, device=DEV), torch.tensor(coff, device=DEV), C)
    # first the documents before `cut`, then the rest pooled into the same bank after their
    # rows (offsets that start at the rows the bank already holds)
    offA, offB = off[:cut + 1], off[cut:] - off[cut]
    coffA = M.msa_chunk_offsets(offA, 64)
    CA = int(coffA[-1])
    coffB = M.msa_chunk_offsets(offB, 64) + CA
    partA = M.msa_pool(K[:off[cut]], V[:off[cut]], Kr[:off[cut]], torch.tensor(offA, device=DEV),
                       torch.tensor(coffA, device=DEV), CA)
    bank = (torch.empty_like(whole[0]), torch.empty_like(whole[1]), partA[2].grown(C))
    bank[0][:CA].copy_(partA[0])
    bank[1][:CA].copy_(partA[1])
    tB = slice(int(off[cut]), T)
    M.msa_pool(K[tB], V[tB], Kr[tB], torch.tensor(offB, device=DEV), torch.tensor(coffB, device=DEV),
               C - CA, out=bank)
    torch.cuda.synchronize()
    assert np.array_equal(np.concatenate([coffA, coffB[1:]]), coff)
    assert torch.equal(whole[0], bank[0]) and torch.equal(whole[1], bank[1]), f"{dtype}: appended K-bar/V-bar differ"
    assert whole[2].equal(bank[2]), f"{dtype}: appended routing keys differ (padding included)"
    if dtype == "bf16":
        Qr = _cpu_randn((40, h, d), 34).to(torch.bfloat16).to(DEV)
        a = route(Qr, [40], whole[2], coff, 8)
        b = route(Qr, [40], bank[2], coff, 8)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])


# ------------------------------------------------------------------------------ routing

def _chunk_counts(n_docs, seed, small_frac=0.4, hi=40):
    rng = np.random.default_rng(seed)
    c = rng.integers(1, hi, size=n_docs)
    c[rng.random(n_docs) < small_frac] = 1          # many one-row documents: many per tile
    return c


ROUTE_CASES = [(lq, path) for lq in (1, 3, 15, 16, 17, 40, 64, 65, 100) for path in ("auto", "dot", "mfma", "batch")]


@pytest.mark.parametrize("lq,path", ROUTE_CASES, ids=[f"lq{a}-{b}" for a, b in ROUTE_CASES])
def test_route_bf16(lq, path):
    say(f"case route bf16 lq={lq} path={path}")
    _route_env(path)
    counts = _chunk_counts(300, 5)
    coff, Krb = random_bank(counts, 8, 128, "bf16", 20)
    Qr = (_cpu_randn((lq, 8, 128), 21) + _cpu_randn((1, 8, 128), 22, 0.5)).to(torch.bfloat16)
    for k in (1, 16):
        ids, sc, ds = route(Qr.to(DEV), [lq], Krb, coff, k)
        o = O.route_doc_scores(f64(Qr), [0, lq], f64(Krb), coff)[0]
        assert_scores_close(ds[0], o, "bf16", f"lq{lq} {path} scores")
        assert_topk_consistent(ids[0], sc[0], ds[0], k, "consistency")
        assert_topk_valid(ids[0], o, k, f"lq{lq} {path} k{k}")


@pytest.mark.parametrize("lq", [1, 8, 20])
def test_route_fp32(lq):
    say(f"case route fp32 lq={lq}")
    counts = _chunk_counts(100, 6)
    coff, Krb = random_bank(counts, 2, 32, "f32", 30)
    Qr = _cpu_randn((lq, 2, 32), 31)
    ids, sc, ds = route(Qr.to(DEV), [lq], Krb, coff, 5)
    o = O.route_doc_scores(f64(Qr), [0, lq], f64(Krb), coff)[0]
    assert_scores_close(ds[0], o, "f32", "fp32 scores")
    assert_topk_valid(ids[0], o, 5, "fp32 topk")


@pytest.mark.parametrize("path", ["auto", "dot", "mfma", "batch"])
def test_route_batched(path):
    say(f"case route batched path={path}")
    _route_env(path)
    counts = _chunk_counts(257, 8)
    coff, Krb = random_bank(counts, 8, 128, "bf16", 40)
    q_lens = [1, 7, 16, 33, 64, 130]
    Qr = _cpu_randn((sum(q_lens), 8, 128), 41).to(torch.bfloat16)
    ids, sc, ds = route(Qr.to(DEV), q_lens, Krb, coff, 16)
    q_off = np.concatenate([[0], np.cumsum(q_lens)])
    o = O.route_doc_scores(f64(Qr), q_off, f64(Krb), coff)
    for b in range(len(q_lens)):
        assert_scores_close(ds[b], o[b], "bf16", f"query {b}")
        assert_topk_consistent(ids[b], sc[b], ds[b], 16, f"query {b}")
        assert_topk_valid(ids[b], o[b], 16, f"query {b}")


@pytest.mark.parametrize("path", ["dot", "mfma", "batch"])
def test_route_batched_parts_share_xcd(path):
    # 4096 rows: 64 parts for the MFMA scan, 128 for the dot scan, so with several queries
    # the workgroups take the XCD-grouped (part, query) order.
    say(f"case route batched, XCD-grouped parts, path={path}")
    _route_env(path)
    counts = _chunk_counts(400, 12, hi=20)
    counts[-1] += 4096 - int(counts.sum())
    assert counts[-1] >= 1 and counts.sum() == 4096
    coff, Krb = random_bank(counts, 8, 128, "bf16", 60)
    for q_lens in ([20, 3, 48], [16] * 8, [1, 17, 2, 64, 5, 30, 16, 7, 40]):
        Qr = _cpu_randn((sum(q_lens), 8, 128), 61 + len(q_lens)).to(torch.bfloat16)
        ids, sc, ds = route(Qr.to(DEV), q_lens, Krb, coff, 8)
        q_off = np.concatenate([[0], np.cumsum(q_lens)])
        o = O.route_doc_scores(f64(Qr), q_off, f64(Krb), coff)
        for b in range(len(q_lens)):
            assert_scores_close(ds[b], o[b], "bf16", f"B={len(q_lens)} query {b}")
            assert_topk_consistent(ids[b], sc[b], ds[b], 8, f"B={len(q_lens)} query {b}")
            assert_topk_valid(ids[b], o[b], 8, f"B={len(q_lens)} query {b}")


def test_route_paths_agree_and_deterministic():
    say("case route dot vs mfma, repeatability")
    counts = _chunk_counts(500, 9)
    coff, Krb = random_bank(counts, 8, 128, "bf16", 50)
    Qr = _cpu_randn((48, 8, 128), 51).to(torch.bfloat16).to(DEV)
    _route_env("mfma")
    a = route(Qr, [48], Krb, coff, 16)
    b = route(Qr, [48], Krb, coff, 16)
    _route_env("dot")
    c = route(Qr, [48], Krb, coff, 16)
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[0], b[0])   # same bits twice
    assert np.max(np.abs(a[2] - c[2])) < 1e-5
    _route_env("batch")
    d = route(Qr, [48], Krb, coff, 16)
    e = route(Qr, [48], Krb, coff, 16)
    assert np.array_equal(d[2], e[2]) and np.array_equal(d[0], e[0])   # atomics merge a max: same bits
    assert np.max(np.abs(a[2] - d[2])) < 1e-5


@pytest.mark.parametrize("heads", [8, 4])
@pytest.mark.parametrize("n_rows", [1, 37, 128, 129, 300])
def test_route_batch_kernel_edges(heads, n_rows):
    # banks smaller than one workgroup's 128 rows, exactly one, one more; documents that
    # cross wave and workgroup boundaries; queries of 1, 0, 16, 17 and 33 tokens
    say(f"case batched scan edges heads={heads} rows={n_rows}")
    _route_env("batch")
    rng = np.random.default_rng(n_rows)
    counts = []
    while sum(counts) < n_rows:
        counts.append(int(min(rng.integers(1, 40), n_rows - sum(counts))))
    coff, Krb = random_bank(np.array(counts), heads, 128, "bf16", 70 + n_rows)
    q_lens = [1, 0, 16, 17, 33]
    Qr = _cpu_randn((sum(q_lens), heads, 128), 71).to(torch.bfloat16)
    q_off = np.concatenate([[0], np.cumsum(q_lens)])
    ds = M.msa_route_scan(Qr.to(DEV), torch.tensor(q_off, dtype=torch.int32, device=DEV), 33, as_keys(Krb),
                          torch.tensor(coff, device=DEV))
    torch.cuda.synchronize()
    ds = ds.cpu().numpy()
    o = O.route_doc_scores(f64(Qr), q_off, f64(Krb), coff)
    for b in range(len(q_lens)):
        if q_lens[b] == 0:
            assert np.all(np.isneginf(ds[b]))
        else:
            assert_scores_close(ds[b], o[b], "bf16", f"rows {n_rows} query {b}")


def _scan_parts(coff, parts):
    """Host copy of the streaming scan's document-aligned split: part p starts at the first
    document whose first row is at or after p * C / P."""
    C = int(coff[-1])
    starts = [int(np.searchsorted(coff, C * p // parts, side="left")) for p in range(parts)] + [len(coff) - 1]
    return [(starts[p], starts[p + 1]) for p in range(parts)]


def _window_crossings(coff, parts, win_rows):
    """Documents whose rows cross a score window of the MFMA scan (windows of win_rows rows
    from the first 16-row tile of each part), and those spanning three windows or more."""
    crossing, three = 0, 0
    for d0, d1 in parts:
        base = (int(coff[d0]) // 16) * 16
        w_first = (coff[d0:d1] - base) // win_rows
        w_last = (coff[d0 + 1:d1 + 1] - 1 - base) // win_rows
        crossing += int(np.sum(w_last > w_first))
        three += int(np.sum(w_last - w_first >= 2))
    return crossing, three


@pytest.mark.parametrize("h_r", [1, 2])
@pytest.mark.parametrize("with_rows", [False, True], ids=["scores", "rows"])
def test_route_scan_window_carry(h_r, with_rows):
    # A bank of 1.1M rows: each of the scan's 256 parts holds several score windows (2,048
    # rows, 1,024 with row outputs), so documents cross window boundaries and their running
    # maximum is carried from one window to the next.  Documents of 4,096 to 9,000 rows
    # span three windows or more.
    say(f"case route scan window carry h_r={h_r} rows={with_rows}")
    _route_env("mfma")
    rng = np.random.default_rng(300 + h_r)
    counts = rng.integers(1, 48, size=46_000)
    counts[[100, 20_000, 30_000, 45_000]] = [9000, 8193, 4097, 4096]
    counts[-1] += max(0, 1_100_000 - int(counts.sum()))
    coff, Krb = random_bank(counts, h_r, 32, "bf16", 310 + h_r)
    C = int(coff[-1])
    # the launch takes 256 parts here: check on the host that the carry is reached
    crossing, three = _window_crossings(coff, _scan_parts(coff, 256), 1024 if with_rows else 2048)
    assert crossing >= 200 and three >= 4, (crossing, three)
    say(f"  {len(counts)} docs, {C} rows; {crossing} documents cross a window, {three} span three or more")
    q_lens = [64, 5]
    Qr = (_cpu_randn((sum(q_lens), h_r, 32), 320) + _cpu_randn((1, h_r, 32), 321, 0.5)).to(torch.bfloat16)
    q_off = np.concatenate([[0], np.cumsum(q_lens)])
    q_off_d = torch.tensor(q_off, dtype=torch.int32, device=DEV)
    coff_d = torch.tensor(coff, device=DEV)
    rows = None
    if with_rows:
        rows = (torch.empty((2, C), dtype=torch.float32, device=DEV), torch.empty((2, C), dtype=torch.int32, device=DEV))
    # one call per query (a single query keeps the plain part order), then both together
    keys = as_keys(Krb)
    per_q = []
    for b in range(2):
        one = torch.tensor([0, q_lens[b]], dtype=torch.int32, device=DEV)
        per_q.append(M.msa_route_scan(Qr[q_off[b]:q_off[b + 1]].to(DEV), one, q_lens[b], keys, coff_d).cpu().numpy()[0])
    Qr_d = Qr.to(DEV)
    ds = M.msa_route_scan(Qr_d, q_off_d, max(q_lens), keys, coff_d, rows=rows)
    ids, sc = M.msa_topk(ds, 16)
    torch.cuda.synchronize()
    ds, ids, sc = ds.cpu().numpy(), ids.cpu().numpy(), sc.cpu().numpy()
    o = oracle_doc_scores_all(Qr, q_off, Krb, coff, block=65536, what="window carry")
    for b in range(2):
        assert_scores_close(per_q[b], o[b], "bf16", f"query {b} alone, every document")
        assert_scores_close(ds[b], o[b], "bf16", f"query {b} batched, every document")
        assert_topk_consistent(ids[b], sc[b], ds[b], 16, f"query {b}")
        assert_topk_valid(ids[b], o[b], 16, f"query {b}")
    if with_rows:
        rs, ra = rows[0].cpu().numpy(), rows[1].cpu().numpy()
        big = [int(x) for x in np.nonzero(counts >= 4096)[0]]
        for b in range(2):
            Qb = f64(Qr[q_off[b]:q_off[b + 1]])
            for d in big:
                r0, r1 = int(coff[d]), int(coff[d + 1])
                o_rows = O.token_chunk_scores(Qb, f64(Krb[r0:r1]))          # [Lq, rows]
                assert_scores_close(rs[b, r0:r1], o_rows.max(axis=0), "bf16", f"query {b} doc {d} row scores")
                # the recorded token reaches its row's maximum within twice the score bar
                got = o_rows[ra[b, r0:r1], np.arange(r1 - r0)]
                best = o_rows.max(axis=0)
                assert np.all(best - got <= 2 * 2e-3 * np.maximum(np.abs(best), 1e-3)), f"query {b} doc {d} row tokens"


def test_topk_ties_and_small_banks():
    say("case top-k ties, k > N, single document")
    # documents 3 and 7 duplicate documents 1 and 2: equal scores, lower id first
    counts = np.array([2, 3, 1, 3, 4, 2, 5, 1])
    coff, Krb = random_bank(counts, 8, 128, "bf16", 60)
    Krb[coff[3]:coff[4]] = Krb[coff[1]:coff[2]]
    Krb[coff[7]:coff[8]] = Krb[coff[2]:coff[3]]
    Qr = _cpu_randn((20, 8, 128), 61).to(torch.bfloat16)
    ids, sc, ds = route(Qr.to(DEV), [20], Krb, coff, 12)
    assert ds[0][1] == ds[0][3] and ds[0][2] == ds[0][7]
    order = list(ids[0][:8])
    assert order.index(1) < order.index(3) and order.index(2) < order.index(7)
    assert list(ids[0][8:]) == [-1] * 4 and np.all(np.isneginf(sc[0][8:]))
    o = O.route_doc_scores(f64(Qr), [0, 20], f64(Krb), coff)[0]
    assert_topk_valid(ids[0], o, 12, "ties")
    coff1, Krb1 = random_bank([3], 8, 128, "bf16", 62)
    ids1, sc1, _ = route(Qr.to(DEV), [20], Krb1, coff1, 4)
    assert list(ids1[0]) == [0, -1, -1, -1]


def test_route_zero_vectors():
    say("case route zero-norm rows")
    counts = np.array([2, 2, 2])
    coff, Krb = random_bank(counts, 8, 128, "bf16", 70)
    Krb[1, 3] = 0
    Qr = _cpu_randn((16, 8, 128), 71).to(torch.bfloat16)
    Qr[5, 2] = 0
    ids, sc, ds = route(Qr.to(DEV), [16], Krb, coff, 3)
    o = O.route_doc_scores(f64(Qr), [0, 16], f64(Krb), coff)[0]
    assert np.all(np.isfinite(ds[0]))
    assert_scores_close(ds[0], o, "bf16", "zero rows")


# ------------------------------------------------------------------------------ attention

ATTN_CASES = [
    # (name, dtype, hq, hkv, d, q_lens, extra_kv, k)
    ("prefill64", "bf16", 32, 8, 128, [64], 0, 16),
    ("decode", "bf16", 32, 8, 128, [1], 40, 16),
    ("batch_ragged", "bf16", 32, 8, 128, [1, 16, 37, 64, 130], 3, 8),
    ("gqa2_d64", "bf16", 8, 4, 64, [20, 5], 7, 4),
    # row blocks of 32, 64 and 128 query rows (2, 4 and 8 waves of one 16-row tile)
    ("rows32_d128", "bf16", 32, 8, 128, [8], 5, 6),
    ("rows64_d128", "bf16", 32, 8, 128, [16, 3], 2, 6),
    ("rows128_d128", "bf16", 32, 8, 128, [32, 7], 0, 6),
    ("d32", "bf16", 4, 2, 32, [9], 0, 3),
    # a query with no tokens (two local keys, nothing attends) between two others
    ("empty_query", "bf16", 8, 2, 64, [5, 0, 7], 2, 4),
    ("fp32_tiny", "f32", 4, 2, 32, [8, 3], 2, 2),
    ("fp32_d128", "f32", 8, 2, 128, [5], 1, 3),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention(case):
    name, dtype, hq, hkv, d, q_lens, extra, k = case
    say(f"case attention {name}")
    counts = _chunk_counts(60, 12, small_frac=0.2, hi=30)
    coff, Kb = random_bank(counts, hkv, d, dtype, 80, doc_std=1.0)
    _, Vb = random_bank(counts, hkv, d, dtype, 82, doc_std=1.0)
    rng = np.random.default_rng(83)
    B = len(q_lens)
    ids = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        keff = k if b % 2 == 0 else max(1, k - 2)      # some queries with unused slots
        ids[b, :keff] = rng.choice(len(counts), size=keff, replace=False)
    kv_lens = [q + extra for q in q_lens]
    Q = _cpu_randn((sum(q_lens), hq, d), 84).to(_dt(dtype))
    Kl = _cpu_randn((sum(kv_lens), hkv, d), 85).to(_dt(dtype))
    Vl = _cpu_randn((sum(kv_lens), hkv, d), 86).to(_dt(dtype))
    q_off = np.concatenate([[0], np.cumsum(q_lens)])
    kv_off = np.concatenate([[0], np.cumsum(kv_lens)])
    args = (Q.to(DEV), Kl.to(DEV), Vl.to(DEV), torch.tensor(q_off, dtype=torch.int32, device=DEV),
            torch.tensor(kv_off, dtype=torch.int32, device=DEV), max(q_lens),
            torch.tensor(ids, device=DEV), torch.tensor(coff, device=DEV))
    out = M.msa_sparse_attn(*args, Kb, Vb, rope_base=1e6)
    torch.cuda.synchronize()
    ref = O.sparse_attn(f64(Q), f64(Kl), f64(Vl), q_off, kv_off, ids, coff, f64(Kb), f64(Vb), 1e6)
    err = assert_attn_close(out, ref, dtype, name)
    say(f"  max abs err {err:.3g}")
    if dtype == "bf16":
        # the same bank read from pinned host memory gives the same bits
        out_h = M.msa_sparse_attn(*args, Kb.cpu().pin_memory(), Vb.cpu().pin_memory(), rope_base=1e6)
        out_2 = M.msa_sparse_attn(*args, Kb, Vb, rope_base=1e6)
        torch.cuda.synchronize()
        assert torch.equal(out_h, out) and torch.equal(out_2, out)


def test_attention_max_k():
    # k = 1024, the largest the library takes: 1,100 documents of one or two rows, so every
    # query's memory spans over a thousand documents (the document table is built 64 ids at a
    # time, and a key's document is found through all eleven lifting steps); the second query
    # leaves its last 100 slots unused, as msa_route_topk does when fewer documents qualify
    say("case attention k = 1024")
    rng = np.random.default_rng(95)
    counts = rng.integers(1, 3, size=1100)
    coff, Kb = random_bank(counts, 2, 64, "bf16", 96, doc_std=1.0)
    _, Vb = random_bank(counts, 2, 64, "bf16", 97, doc_std=1.0)
    k = 1024
    ids = np.full((2, k), -1, dtype=np.int32)
    ids[0] = rng.choice(len(counts), size=k, replace=False)
    ids[1, :k - 100] = rng.choice(len(counts), size=k - 100, replace=False)
    q_lens, kv_lens = [12, 5], [14, 5]
    Q = _cpu_randn((sum(q_lens), 8, 64), 98).to(torch.bfloat16)
    Kl = _cpu_randn((sum(kv_lens), 2, 64), 99).to(torch.bfloat16)
    Vl = _cpu_randn((sum(kv_lens), 2, 64), 100).to(torch.bfloat16)
    q_off = np.concatenate([[0], np.cumsum(q_lens)])
    kv_off = np.concatenate([[0], np.cumsum(kv_lens)])
    out = M.msa_sparse_attn(Q.to(DEV), Kl.to(DEV), Vl.to(DEV), torch.tensor(q_off, dtype=torch.int32, device=DEV),
                            torch.tensor(kv_off, dtype=torch.int32, device=DEV), max(q_lens),
                            torch.tensor(ids, device=DEV), torch.tensor(coff, device=DEV), Kb, Vb, rope_base=1e6)
    torch.cuda.synchronize()
    ref = O.sparse_attn(f64(Q), f64(Kl), f64(Vl), q_off, kv_off, ids, coff, f64(Kb), f64(Vb), 1e6)
    err = assert_attn_close(out, ref, "bf16", "k = 1024")
    say(f"  max abs err {err:.3g}")


def test_attention_scale_argument():
    say("case attention explicit scale")
    coff, Kb = random_bank([3, 2], 2, 64, "bf16", 90)
    _, Vb = random_bank([3, 2], 2, 64, "bf16", 91)
    Q = _cpu_randn((4, 4, 64), 92).to(torch.bfloat16)
    Kl = _cpu_randn((4, 2, 64), 93).to(torch.bfloat16)
    Vl = _cpu_randn((4, 2, 64), 94).to(torch.bfloat16)
    ids = np.array([[1, 0]], dtype=np.int32)
    out = M.msa_sparse_attn(Q.to(DEV), Kl.to(DEV), Vl.to(DEV), torch.tensor([0, 4], dtype=torch.int32, device=DEV),
                            torch.tensor([0, 4], dtype=torch.int32, device=DEV), 4, torch.tensor(ids, device=DEV),
                            torch.tensor(coff, device=DEV), Kb, Vb, rope_base=1e4, scale=0.05)
    torch.cuda.synchronize()
    ref = O.sparse_attn(f64(Q), f64(Kl), f64(Vl), [0, 4], [0, 4], ids, coff, f64(Kb), f64(Vb), 1e4, scale=0.05)
    assert_attn_close(out, ref, "bf16", "scale 0.05")


# ------------------------------------------------------------------------------ steps alone

# (65_536, 64): 8 slices x 64 = 512 candidates, the largest merge placed by rank;
# (100_003, 64): 832 candidates, merged by the bitonic sort
@pytest.mark.parametrize("n,k", [(1, 1), (5, 8), (1000, 16), (47_000, 16), (100_003, 32), (5000, 1024),
                                 (65_536, 64), (100_003, 64)])
def test_topk_alone_exact(n, k):
    say(f"case top-k alone n={n} k={k}")
    rng = np.random.default_rng(n + k)
    sc = np.round(rng.standard_normal((3, n)), 2).astype(np.float32)   # many ties
    sc[0, : min(n, 7)] = 0.0
    sc[0, min(n, 7): min(n, 14)] = -0.0                                  # -0.0 ties +0.0
    sc[2] = -np.inf
    sc[2, n // 2] = 1.0
    ids, top = M.msa_topk(torch.tensor(sc, device=DEV), k)
    torch.cuda.synchronize()
    ids, top = ids.cpu().numpy(), top.cpu().numpy()
    keff = min(k, n)
    for b in range(3):
        key = np.where(sc[b] == 0, 0.0, sc[b]).astype(np.float64)
        order = np.lexsort((np.arange(n), -key))[:keff]
        assert np.array_equal(ids[b, :keff], order), f"row {b}"
        assert np.array_equal(top[b, :keff], np.where(sc[b][order] == 0, 0.0, sc[b][order]))
        assert np.all(ids[b, keff:] == -1)


@pytest.mark.parametrize("n,k", [(8192, 16), (47_000, 16), (30_000, 100)])
def test_topk_narrow_band(n, k):
    # continuous scores inside a narrow band share their sign, exponent and leading mantissa
    # bits, so the radix select starts below them and needs several passes; exact against a
    # sort of the same float32 values
    say(f"case top-k narrow band n={n} k={k}")
    rng = np.random.default_rng(n + 3 * k)
    sc = (0.3 + 1e-4 * rng.random((2, n))).astype(np.float32)
    sc[1, ::7] = np.float32(0.3)  # a tie run at the band's low edge
    ids, top = M.msa_topk(torch.tensor(sc, device=DEV), k)
    torch.cuda.synchronize()
    ids, top = ids.cpu().numpy(), top.cpu().numpy()
    for b in range(2):
        order = np.lexsort((np.arange(n), -sc[b].astype(np.float64)))[:k]
        assert np.array_equal(ids[b], order), f"row {b}"
        assert np.array_equal(top[b], sc[b][order])


def test_route_scan_alone_and_empty_query():
    say("case route scan alone, empty query")
    counts = _chunk_counts(120, 13)
    coff, Krb = random_bank(counts, 8, 128, "bf16", 100)
    q_lens = [20, 0, 5]
    Qr = _cpu_randn((sum(q_lens), 8, 128), 101).to(torch.bfloat16)
    q_off = np.concatenate([[0], np.cumsum(q_lens)])
    for path in ("auto", "dot", "mfma", "batch"):
        _route_env(path)
        ds = M.msa_route_scan(Qr.to(DEV), torch.tensor(q_off, dtype=torch.int32, device=DEV), 20, as_keys(Krb),
                              torch.tensor(coff, device=DEV))
        ids, sc = M.msa_topk(ds, 4)
        torch.cuda.synchronize()
        ds = ds.cpu().numpy()
        o1 = O.route_doc_scores(f64(Qr), q_off[[1, 2]], f64(Krb), coff)[0]
        assert np.all(np.isneginf(ds[1])) and np.all(np.isneginf(o1)), path
        assert list(ids[1].cpu().numpy()) == list(O.topk_docs(o1, 4)[0]) == [0, 1, 2, 3]
        o = O.route_doc_scores(f64(Qr), q_off[[0, 1]], f64(Krb), coff)[0]
        assert_scores_close(ds[0], o, "bf16", f"{path} q0")
        o2 = O.route_doc_scores(f64(Qr), q_off[[2, 3]] , f64(Krb), coff)[0]
        assert_scores_close(ds[2], o2, "bf16", f"{path} q2")
