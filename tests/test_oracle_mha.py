"""Pins of the oracle's multi-head attention decode (the baseline the latent
cache replaces: [LAT] §2.1 textbook attention over a per-head K/V cache).
Against library attention (torch SDPA in float64); against the MLA oracle on
explicitly rebuilt keys and values ([V2] §2.1: K = W_UK c, V = W_UV c, with
the shared k_R concatenated, §2.3), which ties the two oracles together;
closed forms (one token, zero query, empty sequence)."""

import numpy as np
import pytest
import torch

import oracle
import synth


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("dq,dv", [(128, 128), (192, 128), (16, 8)])
def test_matches_library_attention(dq, dv):
    B, H, S = 3, 4, 37
    q, k, v = _rand(1, B, H, dq), _rand(2, B, H, S, dq), _rand(3, B, H, S, dv)
    lens = np.array([37, 1, 20], np.int32)
    o, lse = oracle.mha_decode(q, k, v, "f64", lens)
    for b in range(B):
        L = lens[b]
        qt = torch.from_numpy(q[b][:, None, :])
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, torch.from_numpy(k[b, :, :L]), torch.from_numpy(v[b, :, :L]))
        assert np.allclose(o[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)
        s = np.einsum("hd,htd->ht", q[b], k[b, :, :L]) / np.sqrt(dq)
        assert np.allclose(lse[b], np.log(np.exp(s).sum(-1)), rtol=0, atol=1e-12)


def test_mla_is_mha_on_rebuilt_keys_and_values():
    """The naive MLA oracle equals this MHA oracle run on the keys [W_UK c; k_R]
    and values W_UV c rebuilt from the latent cache (d_qk = 192, d_v = 128)."""
    wl = synth.workload("dsv2_b32_l2k").with_(batch=2, heads=4, seq_len=None,
                                             seed=synth.workloads.BASE_SEED + 140)
    inp = synth.make_inputs(wl, lengths=[50, 7])
    dl, dr = wl.d_latent, wl.d_rope
    rows = oracle.decode_array(inp.rows, "bf16")
    wuk = oracle.decode_array(inp.w_uk, "bf16")       # [H, d_nope, d_latent]
    wuv = oracle.decode_array(inp.w_uv, "bf16")       # [H, d_v, d_latent]
    qn = oracle.decode_array(inp.q_nope, "bf16")
    qr = oracle.decode_array(inp.q_rope, "bf16")
    stride = 50
    K = np.zeros((2, 4, stride, 192))
    V = np.zeros((2, 4, stride, 128))
    for b, L in enumerate([50, 7]):
        c = rows[[inp.row_index(b, t) for t in range(L)]]  # [L, 576]
        for h in range(4):
            K[b, h, :L, :128] = c[:, :dl] @ wuk[h].T
            K[b, h, :L, 128:] = c[:, dl:dl + dr]
            V[b, h, :L] = c[:, :dl] @ wuv[h].T
    q = np.concatenate([qn, qr], axis=-1)
    o_mha, lse_mha = oracle.mha_decode(q, K, V, "f64", np.array([50, 7], np.int32),
                                       scale=1.0 / np.sqrt(192.0))
    o_mla, lse_mla, _ = oracle.decode_inputs(inp)
    assert np.allclose(o_mha.reshape(-1, 128), o_mla, rtol=0, atol=1e-10)
    assert np.allclose(lse_mha.ravel(), lse_mla, rtol=0, atol=1e-10)


def test_closed_forms():
    q, k, v = _rand(4, 1, 2, 16), _rand(5, 1, 2, 9, 16), _rand(6, 1, 2, 9, 8)
    o, lse = oracle.mha_decode(q, k, v, "f64", np.array([1], np.int32))
    assert np.allclose(o[0], v[0, :, 0], rtol=0, atol=1e-15)
    assert np.allclose(lse[0], np.einsum("hd,hd->h", q[0], k[0, :, 0]) / 4.0, atol=1e-14)
    o, _ = oracle.mha_decode(np.zeros_like(q), k, v, "f64", np.array([9], np.int32))
    assert np.allclose(o[0], v[0].mean(axis=1), rtol=0, atol=1e-14)
    o, lse = oracle.mha_decode(q, k, v, "f64", np.array([0], np.int32))
    assert np.all(o == 0) and np.all(lse == -np.inf)


@pytest.mark.parametrize("H,Hkv", [(8, 2), (8, 1), (6, 3), (4, 4)])
def test_gqa_matches_library_grouped_attention(H, Hkv):
    """Grouped-query attention ([LAT] §2.2): torch SDPA in float64 with each
    key/value head repeated for the G = H / H_kv consecutive query heads of
    its group (repeat_interleave)."""
    B, S, dq, dv = 3, 29, 16, 12
    q, k, v = _rand(7, B, H, dq), _rand(8, B, Hkv, S, dq), _rand(9, B, Hkv, S, dv)
    lens = np.array([29, 1, 11], np.int32)
    o, lse = oracle.gqa_decode(q, k, v, "f64", lens)
    G = H // Hkv
    for b in range(B):
        L = lens[b]
        kk = torch.from_numpy(k[b, :, :L]).repeat_interleave(G, dim=0)
        vv = torch.from_numpy(v[b, :, :L]).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b][:, None, :]), kk.contiguous(), vv.contiguous())
        assert np.allclose(o[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)
        s = torch.einsum("hd,htd->ht", torch.from_numpy(q[b]), kk).numpy() / np.sqrt(dq)
        assert np.allclose(lse[b], np.log(np.exp(s).sum(-1)), rtol=0, atol=1e-12)
    if Hkv == H:  # one key/value head per query head: the MHA oracle
        o2, l2 = oracle.mha_decode(q, k, v, "f64", lens)
        assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def test_mqa_is_mla_with_identity_up_projections():
    """One key/value head shared by all query heads (H_kv = 1) on keys
    [c[:128] | k_R] and values c[:128] equals the naive MLA oracle with W_UK =
    W_UV = [I | 0] ([V2] §2.1: then every head rebuilds the same key and value
    from the latent)."""
    wl = synth.workload("dsv2_b32_l2k").with_(batch=2, heads=4, seq_len=None,
                                             seed=synth.workloads.BASE_SEED + 141)
    inp = synth.make_inputs(wl, lengths=[40, 3])
    eye = np.zeros((4, 128, 512), np.float64)
    eye[:, np.arange(128), np.arange(128)] = 1.0
    rows = oracle.decode_array(inp.rows, "bf16")
    qn = oracle.decode_array(inp.q_nope, "bf16")
    qr = oracle.decode_array(inp.q_rope, "bf16")
    o_mla, lse_mla, _ = oracle.decode(qn, qr, "f64", eye, eye, "f64", rows, "f64", inp.seq_lens,
                                      seq_stride=inp.seq_stride)
    K = np.zeros((2, 1, 40, 192))
    V = np.zeros((2, 1, 40, 128))
    for b, L in enumerate([40, 3]):
        c = rows[[inp.row_index(b, t) for t in range(L)]]
        K[b, 0, :L, :128] = c[:, :128]
        K[b, 0, :L, 128:] = c[:, 512:]
        V[b, 0, :L] = c[:, :128]
    o, lse = oracle.gqa_decode(np.concatenate([qn, qr], -1), K, V, "f64",
                               np.array([40, 3], np.int32), scale=1 / np.sqrt(192.0))
    assert np.allclose(o.reshape(-1, 128), o_mla, rtol=0, atol=1e-12)
    assert np.allclose(lse.ravel(), lse_mla, rtol=0, atol=1e-12)
