"""GPU: the MHA baseline decode (mla_mha_decode) through the C ABI against the
oracle's textbook attention, with ragged and empty sequences and tails that
cover partial steps and idle waves."""

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import oracle
from tests.mla_cases import rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _log(msg):
    print(msg, flush=True)


def _inputs(seed, B, H, stride):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(B, H, 128, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, stride, 128, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, stride, 128, device="cuda", generator=g).to(torch.bfloat16)
    return q, k, v


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("o_dt", [torch.bfloat16, torch.float32])
def test_mha_small_every_output(o_dt):
    lens = [0, 1, 17, 63, 64, 65, 300, 1000]
    B, H, stride = len(lens), 16, 1024
    q, k, v = _inputs(11, B, H, stride)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = torch.empty(B, H, 128, dtype=o_dt, device="cuda")
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    _log(f"mha small o={o_dt}")
    mla.mla_mha_decode(q, k, v, seq, max(lens), o, lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.mha_decode(_bits(q), _bits(k), _bits(v), "bf16", np.array(lens, np.int32))
    tol = 2e-2 if o_dt == torch.bfloat16 else 1e-4
    got = o.float().cpu().numpy()
    e = rel_err(got.reshape(-1, 128), o_ref.reshape(-1, 128))
    fin = np.isfinite(lse_ref)
    el = np.abs(lse.cpu().numpy()[fin] - lse_ref[fin]).max()
    _log(f"  err o {e:.2e} lse {el:.2e}")
    assert e <= tol and el <= tol
    assert np.all(got[0] == 0) and np.all(np.isneginf(lse.cpu().numpy()[0]))


def test_mha_dsv2_heads_sampled():
    """128 heads, L = 2048, the geometry of the MLA headline workload (at batch
    4); sampled (b, h) pairs against the oracle."""
    B, H, L = 4, 128, 2048
    q, k, v = _inputs(12, B, H, L)
    seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o = torch.empty(B, H, 128, dtype=torch.bfloat16, device="cuda")
    _log("mha 128 heads, L=2048")
    mla.mla_mha_decode(q, k, v, seq, L, o)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    pairs = [(0, 0), (1, 63), (2, 100), (3, 127)]
    for b, h in pairs:
        o_ref, _ = oracle.mha_decode(_bits(q[b:b + 1, h:h + 1]), _bits(k[b:b + 1, h:h + 1]),
                                     _bits(v[b:b + 1, h:h + 1]), "bf16", np.array([L], np.int32))
        assert rel_err(got[b, h], o_ref[0, 0]) <= 2e-2, (b, h)


@pytest.mark.parametrize("Hkv", [1, 8, 16, 128])
def test_gqa_every_output(Hkv):
    """Grouped-query decode at 128 query heads and 1 / 8 / 16 / 128 key/value
    heads (multi-query ... multi-head), ragged and empty sequences, every
    output against the oracle."""
    lens = [0, 1, 33, 700, 2048]
    B, H, stride = len(lens), 128, 2048
    g = torch.Generator(device="cuda").manual_seed(40 + Hkv)
    q = torch.randn(B, H, 128, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, stride, 128, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, stride, 128, device="cuda", generator=g).to(torch.bfloat16)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = torch.empty(B, H, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    _log(f"gqa kv_heads={Hkv}")
    mla.mla_gqa_decode(q, k, v, seq, max(lens), o, lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.gqa_decode(_bits(q), _bits(k), _bits(v), "bf16",
                                       np.array(lens, np.int32))
    got = o.cpu().numpy()
    e = rel_err(got.reshape(-1, 128), o_ref.reshape(-1, 128))
    fin = np.isfinite(lse_ref)
    el = np.abs(lse.cpu().numpy()[fin] - lse_ref[fin]).max()
    _log(f"  err o {e:.2e} lse {el:.2e}")
    assert e <= 1e-4 and el <= 1e-4
    assert np.all(got[0] == 0) and np.all(np.isneginf(lse.cpu().numpy()[0]))
