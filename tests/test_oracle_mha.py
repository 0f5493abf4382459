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
