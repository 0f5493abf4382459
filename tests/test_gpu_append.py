"""GPU: mla_cache_append through the C ABI against the oracle's cache append,
bit for bit (codes, bf16/fp32 bits and row scales), then a decode step over
the appended cache against the oracle."""

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import oracle
import synth
from synth.encode import f32_to_bf16_bits
from tests.mla_cases import TOL, DeviceInputs, check_against_oracle, run_step

pytestmark = pytest.mark.gpu

DL, DR, W = 512, 64, 576
NP = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}
TT = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _log(msg):
    print(msg, flush=True)


def _new_rows(seed, B):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, W)).astype(np.float32)
    x *= (10.0 ** r.uniform(-4, 4, size=(B, 1))).astype(np.float32)
    x[0] = 0.0                  # all-zero row: the smallest factor, every code 0
    x[1, :8] = -0.0
    u = x.view(np.uint32)       # exact bf16 ties in row 2
    u[2, :32] = (u[2, :32] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    return x


def _to_dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dt == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def _dev_bits(t, dt):
    a = t.cpu()
    if dt == "bf16":
        a = a.view(torch.int16)
    return a.numpy().view(NP[dt])


CASES = [(c, s, p) for c in ("f32", "bf16", "fp8") for s in ("f32", "bf16") for p in (False, True)]


@pytest.mark.parametrize("cache_dt,src_dt,paged", CASES)
def test_append_matches_oracle_bitwise(cache_dt, src_dt, paged):
    B, stride, max_pages, ps = 37, 40, 3, 64
    r = np.random.default_rng(1000 + 10 * ["f32", "bf16", "fp8"].index(cache_dt) + paged)
    x = _new_rows(7 + paged, B)
    src = x if src_dt == "f32" else f32_to_bf16_bits(x)
    if paged:
        n_rows = B * max_pages * ps
        bt = r.permutation(B * max_pages).astype(np.int32).reshape(B, max_pages)
        bt[3, 1] = -1                                       # an unmapped page
        pos = r.integers(0, max_pages * ps, size=B).astype(np.int32)
        pos[:6] = [0, 63, 64, 191, 192, -5]                 # 192: past the capacity
        pos[3] = 70                                         # falls in the unmapped page
    else:
        n_rows = B * stride
        bt = None
        pos = r.integers(0, stride, size=B).astype(np.int32)
        pos[:6] = [0, stride - 1, stride, -1, 17, 5]        # stride: past the capacity
    # poison: every row that is not written must keep these bits
    rows = r.integers(0, 256, size=(n_rows, W * np.dtype(NP[cache_dt]).itemsize), dtype=np.uint8)
    rows = rows.view(NP[cache_dt]).copy()
    scale = (r.standard_normal(n_rows).astype(np.float32) if cache_dt == "fp8" else None)

    want_rows, want_scale = rows.copy(), (None if scale is None else scale.copy())
    oracle.cache_append(src[:, :DL], src[:, DL:], src_dt, pos, want_rows, cache_dt,
                        row_scale=want_scale, page_size=ps if paged else 0,
                        seq_stride=0 if paged else stride, block_table=bt)

    d_rows = torch.from_numpy(rows.view(np.uint8).copy()).cuda()
    d_rows = d_rows.view(TT[cache_dt]) if cache_dt != "fp8" else d_rows
    d_scale = None if scale is None else torch.from_numpy(scale.copy()).cuda()
    cache = mla.Cache(rows=d_rows, seq_lens=torch.zeros(B, dtype=torch.int32, device="cuda"),
                      max_seq_len=0, row_scale=d_scale,
                      block_table=None if bt is None else torch.from_numpy(bt).cuda(),
                      seq_stride=0 if paged else stride, page_size=ps if paged else 0)
    geo = mla.Geometry(heads=128)
    _log(f"append cache={cache_dt} src={src_dt} paged={paged} B={B}")
    mla.mla_cache_append(geo, _to_dev(src[:, :DL], src_dt), _to_dev(src[:, DL:], src_dt),
                         torch.from_numpy(pos).cuda(), cache)
    torch.cuda.synchronize()
    got = d_rows.cpu().view(torch.uint8).numpy()
    assert np.array_equal(got, want_rows.view(np.uint8))
    if scale is not None:
        assert np.array_equal(d_scale.cpu().numpy().view(np.uint32), want_scale.view(np.uint32))


@pytest.mark.parametrize("name,paged", [("dsv2_b32_l2k", False), ("paged_b64_ragged", True),
                                        ("fp8_b1_l128k", False)])
def test_decode_after_append(name, paged):
    """Sequences of length L_b + 1 whose last row is (re)written by the append:
    the device cache equals the oracle-appended host cache bit for bit, and a
    decode step over it matches the oracle."""
    lens = [300, 1, 64, 97, 31]
    wl = synth.workload(name).with_(batch=len(lens), seq_len=None, num_splits=3,
                                    seed=synth.workloads.BASE_SEED + 120)
    inp = synth.make_inputs(wl, lengths=[n + 1 for n in lens])
    dev = DeviceInputs(inp)
    # new rows drawn like the cache's own values (N(0,1)): the logits stay in
    # the range the decode tolerances are stated for
    x = np.random.default_rng(31).standard_normal((len(lens), W)).astype(np.float32)
    src = f32_to_bf16_bits(x)
    pos = np.array(lens, np.int32)
    _log(f"decode after append: {name}")
    mla.mla_cache_append(dev.geo, _to_dev(src[:, :DL], "bf16"), _to_dev(src[:, DL:], "bf16"),
                         torch.from_numpy(pos).cuda(), dev.cache)
    oracle.cache_append(src[:, :DL], src[:, DL:], "bf16", pos, inp.rows, wl.cache_dtype,
                        row_scale=inp.row_scale, page_size=wl.page_size,
                        seq_stride=inp.seq_stride, block_table=inp.block_table)
    torch.cuda.synchronize()
    assert np.array_equal(_dev_bits(dev.cache.rows, wl.cache_dtype), inp.rows)
    if inp.row_scale is not None:
        assert np.array_equal(dev.cache.row_scale.cpu().numpy().view(np.uint32),
                              inp.row_scale.view(np.uint32))
    step = run_step(dev, wl.num_splits)
    pairs = [(b, h) for b in range(len(lens)) for h in (0, 77, 127)]
    kind = "fp8" if wl.cache_dtype == "fp8" else "bf16"
    e = check_against_oracle(dev, step, pairs, TOL[kind])
    _log(f"  err o/u/lse = {e}")
