"""The Python binding refuses tensors whose dtype, shape or placement does not match what
the C entry point reads through its pointers, before any pointer reaches the library (no
GPU needed: the checks run on host tensors, and placement is checked after dtype and shape)."""
import pytest
import torch

m = pytest.importorskip("latent_memory_long_amd")
MsaError = m.MsaError

bf, f32, i32, i64 = torch.bfloat16, torch.float32, torch.int32, torch.int64


def z(shape, dt):
    return torch.zeros(shape, dtype=dt)


def keys(C=6, h_r=2, d=32, dt=bf):
    """Routing keys of C rows in the bank layout (host storage: the checks never reach it)."""
    return m.RouteKeys(z((m.msa_krbar_elems(1 if dt == bf else 0, C, h_r, d),), dt), C, h_r, d)


def route_args(**over):
    a = dict(Qr=z((4, 2, 32), bf), q_off=torch.tensor([0, 4], dtype=i32), max_q_len=4,
             Krbar=keys(), chunk_off=torch.tensor([0, 2, 6], dtype=i64))
    a.update(over)
    return a


def attn_args(**over):
    a = dict(Q=z((3, 4, 32), bf), Kloc=z((5, 2, 32), bf), Vloc=z((5, 2, 32), bf),
             q_off=torch.tensor([0, 3], dtype=i32), kv_off=torch.tensor([0, 5], dtype=i32), max_q_len=3,
             topk_ids=torch.tensor([[1, 0]], dtype=i32), chunk_off=torch.tensor([0, 2, 6], dtype=i64),
             Kbar=z((6, 2, 32), bf), Vbar=z((6, 2, 32), bf))
    a.update(over)
    return a


def refused(fn, kw, text):
    with pytest.raises(MsaError) as e:
        fn(**kw)
    assert e.value.status == m.binding.MSA_ERR_INVALID_ARG
    assert text in e.value.message, e.value.message


@pytest.mark.parametrize("over,text", [
    (dict(q_off=torch.tensor([0, 4], dtype=i64)), "q_off has dtype"),
    (dict(chunk_off=torch.tensor([0, 2, 6], dtype=i32)), "chunk_off has dtype"),
    (dict(Qr=z((4, 2, 32), f32)), "Qr has dtype"),
    (dict(Qr=z((4, 3, 32), bf)), "Qr has shape"),
    (dict(Qr=z((4, 2, 64), bf)), "Qr has shape"),
    (dict(Krbar=z((6, 2, 32), bf)), "Krbar must be a RouteKeys"),
    (dict(Krbar=keys(dt=f32)), "Qr has dtype"),
    (dict(Qr=z((2, 4, 32), bf).transpose(0, 1)), "Qr must be contiguous"),
    (dict(), "must be a device tensor"),
])
def test_route_refusals(over, text):
    refused(m.msa_route_scan, route_args(**over), text)
    kw = route_args(**over)
    kw["k"] = 2
    refused(m.msa_route_topk, kw, text)


def test_route_keys_refusals():
    with pytest.raises(MsaError) as e:
        m.RouteKeys(z((6 * 2 * 32,), bf), 6, 2, 32)        # row count, not whole 16-row tiles
    assert "RouteKeys data has shape" in e.value.message
    with pytest.raises(MsaError) as e:
        m.RouteKeys(z((16 * 2 * 32,), torch.float16), 6, 2, 32)
    assert "RouteKeys data has dtype" in e.value.message
    assert m.msa_krbar_elems(1, 17, 2, 32) == 32 * 2 * 32 and m.msa_krbar_elems(0, 17, 2, 32) == 17 * 2 * 32
    assert keys(17).shape == (17, 2, 32) and keys(17).data.numel() == 32 * 64
    with pytest.raises(MsaError):
        m.msa_krbar_elems(1, 5, 2, 48)                        # head dim outside {32, 64, 128}
    # a float32 bank may also be a plain row-major tensor
    refused(m.msa_route_scan, route_args(Qr=z((4, 2, 32), f32), Krbar=z((6, 2, 32), f32)), "must be a device tensor")


def test_route_output_refusals():
    refused(m.msa_route_scan, route_args(out=z((1, 3), f32)), "doc_scores has shape")
    kw = route_args(k=2, out=(z((1, 2), i64), z((1, 2), f32), None))
    refused(m.msa_route_topk, kw, "topk_ids has dtype")


@pytest.mark.parametrize("over,text", [
    (dict(kv_off=torch.tensor([0, 5], dtype=i64)), "kv_off has dtype"),
    (dict(q_off=torch.tensor([0, 3], dtype=i64)), "q_off has dtype"),
    (dict(topk_ids=torch.tensor([[1, 0]], dtype=i64)), "topk_ids has dtype"),
    (dict(topk_ids=torch.tensor([[1, 0], [0, 1]], dtype=i32)), "topk_ids has shape"),
    (dict(chunk_off=torch.tensor([0, 2, 6], dtype=i32)), "chunk_off has dtype"),
    (dict(Vloc=z((4, 2, 32), bf)), "Vloc has shape"),
    (dict(Kloc=z((5, 2, 64), bf), Vloc=z((5, 2, 64), bf)), "Kloc has shape"),
    (dict(Kbar=z((6, 2, 32), f32)), "Kbar has dtype"),
    (dict(Kbar=z((6, 4, 32), bf), Vbar=z((6, 4, 32), bf)), "Kbar has shape"),
    (dict(Vbar=z((5, 2, 32), bf)), "Vbar has shape"),
    (dict(), "must be a device tensor"),
])
def test_attn_refusals(over, text):
    refused(m.msa_sparse_attn, attn_args(**over), text)


def test_attn_backward_refusals():
    kw = attn_args(O=z((3, 4, 32), bf), dO=z((3, 4, 32), f32))
    refused(m.msa_sparse_attn_backward, kw, "dO has dtype")
    kw = attn_args(O=z((3, 4, 32), bf), dO=z((3, 4, 32), bf), dbank=(z((6, 2, 32), bf), z((6, 2, 32), f32)),
                   out=(z((3, 4, 32), f32), z((5, 2, 32), f32), z((5, 2, 32), f32)))
    refused(m.msa_sparse_attn_backward, kw, "dKbar has dtype")


def test_pool_refusals():
    K = z((10, 2, 32), bf)
    base = dict(K=K, V=z((10, 2, 32), bf), Kr=z((10, 1, 32), bf), doc_tok_off=torch.tensor([0, 4, 10], dtype=i64),
                chunk_off=torch.tensor([0, 1, 2], dtype=i64), n_chunks=2)
    refused(m.msa_pool, {**base, "chunk_off": torch.tensor([0, 1, 2], dtype=i32)}, "chunk_off has dtype")
    refused(m.msa_pool, {**base, "doc_tok_off": torch.tensor([0, 4, 10], dtype=i32)}, "doc_tok_off has dtype")
    refused(m.msa_pool, {**base, "V": z((10, 3, 32), bf)}, "V has shape")
    refused(m.msa_pool, {**base, "Kr": z((10, 1, 32), f32)}, "Kr has dtype")
    refused(m.msa_pool, {**base, "chunk_off": torch.tensor([0, 1], dtype=i64)}, "chunk_off has shape")
    refused(m.msa_pool, base, "must be a device tensor")


def test_topk_and_loss_refusals():
    refused(m.msa_topk, dict(doc_scores=z((2, 5), torch.float64), k=2), "doc_scores has dtype")
    refused(m.msa_topk, dict(doc_scores=z((2, 5), f32), k=2), "must be a device tensor")
    refused(m.msa_route_aux_loss, dict(doc_scores=z((2, 5), f32), labels=z((2, 4), f32)), "labels has shape")
    kw = route_args(dD=z((1, 2), f64 := torch.float64))
    refused(m.msa_route_backward, kw, "dD has dtype")


def test_pool_output_refusals():
    K = z((10, 2, 32), bf)
    base = dict(K=K, V=z((10, 2, 32), bf), Kr=z((10, 1, 32), bf), doc_tok_off=torch.tensor([0, 4, 10], dtype=i64),
                chunk_off=torch.tensor([0, 1, 2], dtype=i64), n_chunks=2)
    refused(m.msa_pool, {**base, "out": (z((2, 2, 32), bf), z((2, 2, 32), bf), z((2, 1, 32), bf))},
            "Krbar must be a RouteKeys")
    refused(m.msa_pool, {**base, "out": (z((2, 2, 32), bf), z((2, 2, 32), bf), keys(3, 1, 32))}, "bank buffers hold")
