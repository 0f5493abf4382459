"""GPU parity: the HIP decode path (absorb -> decode -> combine -> up-projection,
called through the C ABI) against the CPU oracle (naive rebuild of K and V,
textbook softmax) on seeded synthetic inputs.

Tolerances: max|o_gpu - o_oracle| <= tol * max|o_oracle| with tol 1e-4 for an
fp32 cache, 2e-2 for bf16 and 6e-2 for an fp8-e4m3 cache; the same bound is
applied to the attention-weighted latent u, and tol as an absolute bound on
lse (natural log).  Cache slots that hold no token are NaN-poisoned by the
generator, so reading one fails the finiteness check.
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_15_amd as mla
import oracle
import synth
from tests.mla_cases import (TOL, DeviceInputs, check_against_oracle, run_step, sample_pairs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")


def _log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- small cases

@pytest.mark.parametrize("splits", [1, 4])
def test_tiny_f32_every_output(splits):
    """fp32 cache, B=1, h=16, L=512: every (b, h) against the oracle at 1e-4."""
    wl = synth.workload("tiny_f32")
    dev = DeviceInputs(synth.make_inputs(wl))
    step = run_step(dev, splits)
    pairs = [(0, h) for h in range(wl.heads)]
    e = check_against_oracle(dev, step, pairs, TOL["f32"])
    _log(f"tiny_f32 S={splits}: err o/u/lse = {e}")


RAGGED = [0, 1, 31, 32, 45, 300, 257]


H64, BAL = mla.KERNEL_H64, mla.KERNEL_H64_BALANCED
# the balanced partition takes 2 splits or more
RAGGED_CASES = ([(h, H64, s) for h in (32, 128, 160, 256) for s in (1, 3, 7)] +
                [(h, BAL, s) for h in (32, 128, 160, 256) for s in (3, 7)])


@pytest.mark.parametrize("heads,kernel,splits", RAGGED_CASES)
def test_ragged_bf16(heads, kernel, splits):
    """bf16, several tiles plus ragged tails, empty and 1-token sequences, on
    the fixed split ranges and on the balanced partition: a partial head group
    (160 = 128 + 32), waves without heads (32), several head groups (256)."""
    wl = synth.workload("dsv2_b32_l2k").with_(batch=len(RAGGED), heads=heads, seq_len=None,
                                             seed=synth.workloads.BASE_SEED + 101)
    dev = DeviceInputs(synth.make_inputs(wl, lengths=RAGGED))
    _log(f"ragged h={heads} kernel={kernel} S={splits}")
    step = run_step(dev, splits, kernel=kernel)
    pairs = [(b, h) for b in range(wl.batch) for h in sorted({0, 1, heads // 2, heads - 1})]
    e = check_against_oracle(dev, step, pairs, TOL["bf16"])
    _log(f"  err o/u/lse = {e}")


@pytest.mark.parametrize("kernel", [H64, BAL])
@pytest.mark.parametrize("part", ["f32", "bf16"])
def test_ragged_fp32_partials(part, kernel):
    """The same bf16 problem with fp32 or bf16 split partials."""
    wl = synth.workload("dsv2_b32_l2k").with_(batch=len(RAGGED), seq_len=None,
                                             seed=synth.workloads.BASE_SEED + 102)
    dev = DeviceInputs(synth.make_inputs(wl, lengths=RAGGED))
    step = run_step(dev, 5, part_dtype=torch.float32 if part == "f32" else torch.bfloat16,
                    kernel=kernel)
    pairs = [(b, h) for b in range(wl.batch) for h in (0, 77, 127)]
    check_against_oracle(dev, step, pairs, TOL["bf16"])


def test_fp8_small():
    """fp8-e4m3 cache with per-row scales, ragged lengths, 3 splits."""
    wl = synth.workload("fp8_b1_l128k").with_(batch=4, seq_len=None,
                                             seed=synth.workloads.BASE_SEED + 103)
    lens = [300, 77, 1, 0]
    dev = DeviceInputs(synth.make_inputs(wl, lengths=lens))
    step = run_step(dev, 3)
    pairs = [(b, h) for b in range(4) for h in (0, 31, 64, 127)]
    e = check_against_oracle(dev, step, pairs, TOL["fp8"])
    _log(f"fp8 small: err o/u/lse = {e}")


def test_fp8_codes_exact():
    """Every finite E4M3 code reaches the PV product unchanged.  With a zero
    query every probability is 1; each sequence holds one row of codes 32
    times (every position of a tile) with a power-of-two scale, so u is that
    row times its scale with no rounding at all, and is compared for equality
    with the oracle's own E4M3 decoder."""
    wl = synth.workload("fp8_b1_l128k").with_(batch=8, seq_len=32, num_splits=1,
                                             seed=synth.workloads.BASE_SEED + 108)
    inp = synth.make_inputs(wl)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    width = inp.rows.shape[1]
    want = []
    for b in range(wl.batch):
        codes = np.roll(np.resize(finite, width), 37 * b)
        scale = np.float32(2.0 ** -(b % 4 + 1))
        for t in range(wl.seq_len):
            r = inp.row_index(b, t)
            inp.rows[r] = codes
            inp.row_scale[r] = scale
        want.append(oracle.decode_array(codes[:wl.d_latent], "fp8") * float(scale))
    dev = DeviceInputs(inp)
    dev.q_nope.zero_()
    dev.q_rope.zero_()
    step = run_step(dev, 1, part_dtype=torch.float32, out_dtype=torch.float32)
    u = step.u_part.float().cpu().numpy()  # [B, 1, H, d_latent]
    for b in range(wl.batch):
        got = u[b, 0].astype(np.float64)
        assert np.array_equal(got, np.broadcast_to(want[b], got.shape)), b


@pytest.mark.parametrize("kernel", [H64, BAL])
def test_paged_matches_contiguous_bitwise(kernel):
    """The same tokens in a shuffled paged pool and in contiguous rows give
    bit-identical partials (the tiles see the same rows in the same order)."""
    base = synth.workload("paged_b64_ragged").with_(batch=6, seed=synth.workloads.BASE_SEED + 104)
    lens = [1, 64, 65, 700, 129, 0]
    paged = DeviceInputs(synth.make_inputs(base, lengths=lens))
    contig = DeviceInputs(synth.make_inputs(base.with_(page_size=0), lengths=lens))
    a = run_step(paged, 3, kernel=kernel)
    b = run_step(contig, 3, kernel=kernel)
    assert torch.equal(a.lse_part, b.lse_part)
    live = torch.isfinite(a.lse_part)  # an empty split's u is not written
    assert torch.equal(a.u_part.view(torch.int16)[live], b.u_part.view(torch.int16)[live])
    assert torch.equal(a.o.view(torch.int16), b.o.view(torch.int16))
    pairs = [(bb, h) for bb in range(6) for h in (0, 127)]
    check_against_oracle(paged, a, pairs, TOL["bf16"])


@pytest.mark.parametrize("kernel", [H64, BAL])
def test_split_count_invariance(kernel):
    """Different split counts give the same result.  With a zero query every
    score is 0, so every probability is exactly 1 in bf16 and u is the plain
    mean of the cached latents: split ranges may only change the fp32
    summation order.  A dropped or repeated token (or tile) shows up as an
    error of order 1/L."""
    wl = synth.workload("dsv2_b32_l2k").with_(batch=3, seq_len=None,
                                             seed=synth.workloads.BASE_SEED + 105)
    dev = DeviceInputs(synth.make_inputs(wl, lengths=[1000, 999, 33]))
    dev.q_nope.zero_()
    dev.q_rope.zero_()
    f32 = torch.float32
    # one split (the balanced partition takes 2 or more: the fixed ranges' result)
    ref = run_step(dev, 1, part_dtype=f32, out_dtype=f32, kernel=H64)
    ref_u = ref.u.clone()
    # u equals the column mean of the cached latents
    rows = dev.cache.rows.float()
    for b, L in enumerate([1000, 999, 33]):
        mean = rows[b * dev.cache.seq_stride: b * dev.cache.seq_stride + L, :512].mean(0)
        assert (ref_u[b] - mean).abs().max().item() < 1e-5
    for s in (2, 3, 7, 32):
        got = run_step(dev, s, part_dtype=f32, out_dtype=f32, kernel=kernel).u
        err = (got - ref_u).abs().max().item()
        _log(f"split invariance kernel={kernel} S={s}: {err:.2e}")
        assert err < 1e-5, (s, err)


def test_split_count_random_inputs():
    """Random scores: split ranges take their own softmax reference, so the
    bf16-rounded probabilities differ (±2^-9 relative each); u is a cancelling
    sum of random latents, so that difference is not averaged away."""
    wl = synth.workload("dsv2_b32_l2k").with_(batch=3, seq_len=1000,
                                             seed=synth.workloads.BASE_SEED + 107)
    dev = DeviceInputs(synth.make_inputs(wl))
    f32 = torch.float32
    ref = run_step(dev, 1, part_dtype=f32, out_dtype=f32).o
    for s in (2, 7, 32):
        got = run_step(dev, s, part_dtype=f32, out_dtype=f32).o
        err = (got - ref).abs().max().item() / ref.abs().max().item()
        assert err < 1e-2, (s, err)


@pytest.mark.parametrize("kernel", [H64, BAL])
def test_max_splits(kernel):
    """The largest split count the ABI takes (1024): 64-token ranges over a
    40,000-token sequence, most ranges of the short and the empty sequence
    empty, and the merge's path for more than 32 splits per sequence."""
    lens = [40000, 33, 0]
    wl = synth.workload("dsv2_b32_l2k").with_(batch=len(lens), seq_len=None,
                                             seed=synth.workloads.BASE_SEED + 108)
    dev = DeviceInputs(synth.make_inputs(wl, lengths=lens))
    _log(f"max splits kernel={kernel}")
    step = run_step(dev, 1024, kernel=kernel)
    pairs = [(b, h) for b in range(len(lens)) for h in (0, 127)]
    e = check_against_oracle(dev, step, pairs, TOL["bf16"])
    _log(f"  err o/u/lse = {e}")


SPIKE_CASES = [("dsv2_b32_l2k", H64), ("dsv2_b32_l2k", BAL), ("fp8_b1_l128k", H64)]


@pytest.mark.parametrize("name,kernel", SPIKE_CASES)
def test_score_spike_recomputes_range(name, kernel):
    """One late token whose RoPE key is 20 q_R of head 0: its score exceeds the
    first tile's reference maximum by far more than the 2^64 slack, so the
    range is computed a second time against its true maximum.  Head 0's output
    is then (nearly) W_UV times that token's latent; every output against the
    oracle."""
    from synth.encode import bf16_bits_to_f32, f32_to_bf16_bits, quantize_rows_e4m3
    lens = [700, 333]
    # past the first tile of the range that holds them, in lanes other than
    # lane 0 of the score layouts of both kernels
    spike = [655, 205]
    wl = synth.workload(name).with_(batch=len(lens), seq_len=None,
                                    seed=synth.workloads.BASE_SEED + 109)
    inp = synth.make_inputs(wl, lengths=lens)
    qr0 = bf16_bits_to_f32(inp.q_rope[:, 0, :])  # [B, 64] query RoPE part of head 0
    for b, t in enumerate(spike):
        r = b * inp.seq_stride + t
        if wl.cache_dtype == "fp8":
            tbl = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
            row = tbl[inp.rows[r]] * inp.row_scale[r]
            row[512:] = 20.0 * qr0[b]
            codes, sc = quantize_rows_e4m3(row[None, :].astype(np.float32))
            inp.rows[r], inp.row_scale[r] = codes[0], sc[0]
        else:
            inp.rows[r, 512:] = f32_to_bf16_bits(20.0 * qr0[b])
    dev = DeviceInputs(inp)
    _log(f"score spike {name} kernel={kernel}")
    kind = "fp8" if wl.cache_dtype == "fp8" else "bf16"
    for splits in ((3,) if kernel == BAL else (1, 3)):
        step = run_step(dev, splits, kernel=kernel)
        pairs = [(b, h) for b in range(len(lens)) for h in (0, 1, 77, 127)]
        e = check_against_oracle(dev, step, pairs, TOL[kind])
        _log(f"  S={splits}: err o/u/lse = {e}")


@pytest.mark.parametrize("name,kernel", [("dsv2_b32_l2k", H64), ("dsv2_b32_l2k", BAL), ("tiny_f32", H64)])
def test_custom_softmax_scale(name, kernel):
    """A caller-given softmax scale (0.05) replaces 1/sqrt(d_nope + d_rope)."""
    wl = synth.workload(name).with_(batch=3, seq_len=None, seed=synth.workloads.BASE_SEED + 110)
    dev = DeviceInputs(synth.make_inputs(wl, lengths=[300, 1, 97]))
    dev.geo.softmax_scale = 0.05
    step = run_step(dev, 3, kernel=kernel)
    pairs = [(b, h) for b in range(3) for h in (0, wl.heads - 1)]
    o_ref, lse_ref, u_ref = oracle.decode_inputs(dev.inp, sel=pairs, want_u=True, scale=0.05)
    kind = "f32" if wl.cache_dtype == "f32" else "bf16"
    o = step.o.float().cpu().numpy()
    lse = step.lse.float().cpu().numpy()
    got = np.stack([o[b, h] for b, h in pairs])
    assert np.abs(got - o_ref).max() <= TOL[kind] * np.abs(o_ref).max()
    assert np.abs(np.array([lse[b, h] for b, h in pairs]) - lse_ref).max() <= TOL[kind]


@pytest.mark.parametrize("name,kernel", [("dsv2_b32_l2k", H64), ("dsv2_b32_l2k", BAL), ("fp8_b1_l128k", H64)])
def test_nan_in_a_read_row_propagates(name, kernel):
    """A NaN in a cached row that is attended (a bf16 NaN, or the E4M3 NaN
    code) makes every output of that sequence NaN (o, u, lse), with one range
    or several; the other sequence is unaffected."""
    lens = [300, 97]
    wl = synth.workload(name).with_(batch=2, seq_len=None, seed=synth.workloads.BASE_SEED + 111)
    inp = synth.make_inputs(wl, lengths=lens)
    # sequence 0, token 150, latent element 3
    inp.rows[150, 3] = 0x7F if wl.cache_dtype == "fp8" else 0x7FC0
    dev = DeviceInputs(inp)
    for splits in ((3,) if kernel == BAL else (1, 3)):
        step = run_step(dev, splits, kernel=kernel)
        o = step.o.float().cpu().numpy()
        u = step.u.float().cpu().numpy()
        lse = step.lse.float().cpu().numpy()
        _log(f"nan row kernel={kernel} S={splits}: nan o/u/lse in seq 0: "
             f"{np.isnan(o[0]).mean():.2f} {np.isnan(u[0]).mean():.2f} {np.isnan(lse[0]).mean():.2f}")
        assert np.isnan(o[0]).all() and np.isnan(u[0]).all() and np.isnan(lse[0]).all()
        if splits > 1:  # the two-call tail (mla_combine, then mla_up_proj) as well
            step.run(dev.q_nope, dev.q_rope, dev.w_uk, dev.w_uv, dev.cache, fused=False)
            torch.cuda.synchronize()
            assert torch.isnan(step.o[0]).all() and torch.isnan(step.u[0].float()).all()
            assert torch.isnan(step.lse[0]).all()
        pairs = [(1, h) for h in (0, 77, 127)]
        o_ref, _, _ = oracle.decode_inputs(dev.inp, sel=pairs)
        got = np.stack([o[b, h] for b, h in pairs])
        tol = TOL["fp8" if wl.cache_dtype == "fp8" else "bf16"]
        assert np.abs(got - o_ref).max() <= tol * np.abs(o_ref).max()


@pytest.mark.parametrize("kernel", [H64, BAL])
def test_large_batch_of_short_sequences(kernel):
    """300 sequences of 0-120 tokens: many 32-sequence tiles in the absorb (the
    staged query rows are replaced tile after tile), many merge workgroups,
    empty and one-token sequences among them."""
    r = np.random.default_rng(112)
    lens = r.integers(0, 121, 300).tolist()
    lens[7], lens[8] = 0, 1
    wl = synth.workload("dsv2_b32_l2k").with_(batch=len(lens), seq_len=None,
                                             seed=synth.workloads.BASE_SEED + 112)
    dev = DeviceInputs(synth.make_inputs(wl, lengths=lens))
    step = run_step(dev, 2, kernel=kernel)
    pairs = [(b, h) for b in (0, 7, 8, 31, 32, 33, 150, 255, 256, 299) for h in (0, 127)]
    e = check_against_oracle(dev, step, pairs, TOL["bf16"])
    _log(f"large batch kernel={kernel}: err o/u/lse = {e}")


def test_repeat_is_deterministic():
    wl = synth.workload("dsv2_b32_l2k").with_(batch=2, seq_len=333,
                                             seed=synth.workloads.BASE_SEED + 106)
    dev = DeviceInputs(synth.make_inputs(wl))
    a = run_step(dev, 4).o.clone()
    b = run_step(dev, 4).o.clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------- full sizes

AUTO = mla.KERNEL_AUTO
F8Q = "fp8 query"  # mla.KERNEL_AUTO with the E4M3 absorbed query
# (workload, tolerance kind, sequences x heads sampled, kernel, parts): the
# sampled sequences are spread from the first to the last (both ends of the
# XCD-aware work order) and the heads over both 64-head groups; a sample whose
# oracle run is long is checked in parts, one test each, on the same run
FULL = [
    ("dsv2_b32_l2k", "bf16", 8, 8, AUTO, 1),
    ("dsv2_b32_l2k", "bf16", 8, 8, BAL, 1),
    ("long_b4_l32k", "bf16", 4, 8, AUTO, 1),
    ("long_b4_l32k", "bf16", 4, 3, H64, 1),
    ("paged_b64_ragged", "bf16", 8, 8, AUTO, 2),
    ("paged_b64_ragged", "bf16", 8, 8, BAL, 2),
    ("fp8_b1_l128k", "fp8", 1, 8, AUTO, 1),
    ("fp8_b8_l128k", "fp8", 8, 8, AUTO, 4),
    # the fp8 absorbed query on the fp8 matrix cores
    ("fp8_b1_l128k", "fp8", 1, 8, F8Q, 1),
    ("fp8_b8_l128k", "fp8", 8, 8, F8Q, 4),
]
FULL_CASES = [(n, k, nb, nh, ker, part, parts) for n, k, nb, nh, ker, parts in FULL
              for part in range(parts)]

_full_cache = {}


def _full_run(name, kernel):
    """inputs and step outputs of one full-size workload, kept for the parts
    of its sample (one workload at a time)"""
    key = (name, kernel)
    if key not in _full_cache:
        _full_cache.clear()
        torch.cuda.empty_cache()
        wl = synth.workload(name)
        _log(f"{name}: generating inputs")
        dev = DeviceInputs(synth.make_inputs(wl))
        _log(f"{name}: running S={wl.num_splits} kernel={kernel}")
        if kernel == F8Q:
            step = run_step(dev, wl.num_splits, fp8_query=True)
        else:
            step = run_step(dev, wl.num_splits, kernel=kernel)
        _full_cache[key] = (dev, step)
    return _full_cache[key]


@pytest.mark.parametrize("name,kind,nb,nh,kernel,part,parts", FULL_CASES)
def test_full_size_sampled(name, kind, nb, nh, kernel, part, parts):
    """Each workload at its full size with its stated split count, checked on a
    spread of (b, h) pairs that the oracle computes one by one."""
    wl = synth.workload(name)
    dev, step = _full_run(name, kernel)
    pairs = sample_pairs(wl.batch, wl.heads, nb, nh)
    pairs = pairs[part * len(pairs) // parts:(part + 1) * len(pairs) // parts]
    _log(f"{name}: part {part + 1}/{parts}, {len(pairs)} pairs")
    e = check_against_oracle(dev, step, pairs, TOL[kind])
    _log(f"{name}: err o/u/lse = {e}")
    o = step.o.float()
    assert torch.isfinite(o).all()


def test_full_size_paged_kernels_agree_on_every_output():
    """The paged ragged workload at full size: the fixed split ranges at the
    workload's split count and at 8 (separate work decompositions) and the
    balanced partition give the same o, u and lse for all 64 x 128 (b, h)
    pairs within the bf16 tolerance."""
    wl = synth.workload("paged_b64_ragged")
    dev, a = _full_run("paged_b64_ragged", AUTO)
    o_a, u_a, l_a = a.o.float().clone(), a.u.float().clone(), a.lse.clone()
    b = run_step(dev, 8, kernel=H64)
    for x, y, what in ((o_a, b.o.float(), "o"), (u_a, b.u.float(), "u")):
        err = ((x - y).abs().max() / y.abs().max()).item()
        _log(f"  {what}: max rel diff {err:.2e}")
        assert err <= TOL["bf16"], what
    assert (l_a - b.lse).abs().max().item() <= TOL["bf16"]
    c = run_step(dev, wl.num_splits, kernel=BAL)  # the balanced partition
    for x, y, what in ((o_a, c.o.float(), "o"), (u_a, c.u.float(), "u")):
        err = ((x - y).abs().max() / y.abs().max()).item()
        _log(f"  balanced {what}: max rel diff {err:.2e}")
        assert err <= TOL["bf16"], what
    assert (l_a - c.lse).abs().max().item() <= TOL["bf16"]
    _full_cache.clear()
