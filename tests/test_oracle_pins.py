"""Pins the CPU oracle to things other than itself.

* library attention (torch SDPA, float64) over explicitly rebuilt K and V, and
  the W = [I | 0] special case that reduces MLA to one-KV-head attention;
* the absorbed form of the DeepSeek V2 MLA page (section 2.3: W_UK folded into
  the query, W_UV applied after the weighted sum) — a different formula that
  must give the same numbers;
* closed forms: one cached token, an all-zero query, one dominant key;
* invariants: a common score shift, token and head permutations, split + merge,
  paged vs contiguous rows, NaN in unread slots, linearity in W_UV, empty
  sequences.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth


def rand_problem(rng, B=2, H=3, L=29, dn=16, dr=8, dl=32, dv=12, lens=None):
    p = dict(
        q_nope=rng.standard_normal((B, H, dn)),
        q_rope=rng.standard_normal((B, H, dr)),
        w_uk=rng.standard_normal((H, dn, dl)) / math.sqrt(dl),
        w_uv=rng.standard_normal((H, dv, dl)) / math.sqrt(dl),
        rows=rng.standard_normal((B * L, dl + dr)),
        lens=np.full(B, L, dtype=np.int32) if lens is None else np.asarray(lens, np.int32),
        stride=L, dims=(dn, dr, dl, dv),
    )
    return p


def run(p, **kw):
    return oracle.decode(p["q_nope"], p["q_rope"], "f64", p["w_uk"], p["w_uv"], "f64",
                         p["rows"], "f64", p["lens"], seq_stride=p["stride"], **kw)


def sdpa_reference(p):
    """torch SDPA (float64) over K_h = [c W_UK[h]^T | k_R], V_h = c W_UV[h]^T."""
    dn, dr, dl, dv = p["dims"]
    B, H = p["q_nope"].shape[:2]
    o = np.zeros((B, H, dv))
    lse = np.zeros((B, H))
    scale = 1.0 / math.sqrt(dn + dr)
    for b in range(B):
        L = int(p["lens"][b])
        rows = torch.from_numpy(p["rows"][b * p["stride"]: b * p["stride"] + L])
        lat, kr = rows[:, :dl], rows[:, dl:]
        for h in range(H):
            K = torch.cat([lat @ torch.from_numpy(p["w_uk"][h]).T, kr], dim=1)
            V = lat @ torch.from_numpy(p["w_uv"][h]).T
            q = torch.cat([torch.from_numpy(p["q_nope"][b, h]), torch.from_numpy(p["q_rope"][b, h])])
            out = torch.nn.functional.scaled_dot_product_attention(
                q[None, None, None], K[None, None].contiguous(), V[None, None].contiguous(),
                scale=scale)
            o[b, h] = out[0, 0, 0].numpy()
            lse[b, h] = torch.logsumexp((K @ q) * scale, dim=0).item()
    return o.reshape(B * H, dv), lse.reshape(B * H)


def assert_close(a, b, rtol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(np.max(np.abs(b)), 1e-300)
    assert np.max(np.abs(a - b)) <= rtol * scale, np.max(np.abs(a - b)) / scale


@pytest.mark.parametrize("dims", [(16, 8, 32, 12), (128, 64, 512, 128)])
def test_matches_library_attention_on_rebuilt_kv(dims):
    rng = np.random.default_rng(10)
    dn, dr, dl, dv = dims
    p = rand_problem(rng, B=2, H=3, L=41, dn=dn, dr=dr, dl=dl, dv=dv)
    o, lse, _ = run(p)
    o_ref, lse_ref = sdpa_reference(p)
    assert_close(o, o_ref)
    assert_close(lse, lse_ref)


def test_identity_weights_reduce_to_one_kv_head_attention():
    # W_UK = W_UV = [I | 0]: every head's key is [c[:dn] ; k_R] and value c[:dv],
    # i.e. attention with a single shared K/V head (library SDPA, float64).
    rng = np.random.default_rng(11)
    dn = dv = 16
    dr, dl, H, L = 8, 32, 4, 23
    p = rand_problem(rng, B=1, H=H, L=L, dn=dn, dr=dr, dl=dl, dv=dv)
    eye = np.zeros((H, dn, dl))
    eye[:, np.arange(dn), np.arange(dn)] = 1.0
    p["w_uk"] = eye.copy()
    p["w_uv"] = eye.copy()
    o, _, _ = run(p)
    rows = torch.from_numpy(p["rows"])
    K = torch.cat([rows[:, :dn], rows[:, dl:]], dim=1)
    V = rows[:, :dv]
    q = torch.from_numpy(np.concatenate([p["q_nope"][0], p["q_rope"][0]], axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[None, :, None], K[None, None].expand(1, H, L, dn + dr).contiguous(),
        V[None, None].expand(1, H, L, dv).contiguous(), scale=1 / math.sqrt(dn + dr))
    assert_close(o, ref[0, :, 0].numpy())


def test_absorbed_form_identity():
    # q~ = W_UK^T q_C ; s_t = scale (q~ . c_t + q_R . k_R,t) ; u = softmax . c ;
    # o = W_UV u  (DeepSeek V2 MLA page, section 2.3 / 4.1)
    rng = np.random.default_rng(12)
    p = rand_problem(rng, B=3, H=4, L=57, dn=128, dr=64, dl=512, dv=128)
    o, lse, u = run(p, want_u=True)
    dn, dr, dl, dv = p["dims"]
    scale = 1 / math.sqrt(dn + dr)
    i = 0
    for b in range(3):
        rows = p["rows"][b * 57:(b + 1) * 57]
        for h in range(4):
            qa = p["w_uk"][h].T @ p["q_nope"][b, h]
            s = scale * (rows[:, :dl] @ qa + rows[:, dl:] @ p["q_rope"][b, h])
            w = np.exp(s - s.max())
            uu = (w / w.sum()) @ rows[:, :dl]
            assert_close(u[i], uu)
            assert_close(o[i], p["w_uv"][h] @ uu)
            assert abs(lse[i] - (s.max() + math.log(w.sum()))) < 1e-12 * abs(lse[i]) + 1e-13
            i += 1


def test_single_token_returns_its_value():
    rng = np.random.default_rng(13)
    p = rand_problem(rng, B=2, H=3, L=1)
    o, _, u = run(p, want_u=True)
    dl = p["dims"][2]
    for b in range(2):
        for h in range(3):
            assert_close(o[b * 3 + h], p["w_uv"][h] @ p["rows"][b, :dl])
            assert_close(u[b * 3 + h], p["rows"][b, :dl])


def test_zero_query_is_uniform_average():
    rng = np.random.default_rng(14)
    L = 31
    p = rand_problem(rng, B=1, H=2, L=L)
    p["q_nope"][:] = 0
    p["q_rope"][:] = 0
    o, lse, u = run(p, want_u=True)
    dl = p["dims"][2]
    mean = p["rows"][:, :dl].mean(axis=0)
    for h in range(2):
        assert_close(u[h], mean)
        assert_close(o[h], p["w_uv"][h] @ mean)
        assert abs(lse[h] - math.log(L)) < 1e-13


def test_one_dominant_key_two_level_weights():
    # q_C = 0 and k_R = 0 except row t* = lam * q_R: scores are 0 except
    # s* = scale * lam |q_R|^2, so o = (e^s* v_t* + sum_{t != t*} v_t) / (e^s* + L - 1)
    rng = np.random.default_rng(15)
    L, ts, lam = 19, 7, 0.3
    p = rand_problem(rng, B=1, H=1, L=L)
    dn, dr, dl, dv = p["dims"]
    p["q_nope"][:] = 0
    p["rows"][:, dl:] = 0
    p["rows"][ts, dl:] = lam * p["q_rope"][0, 0]
    o, lse, _ = run(p)
    sstar = lam * float(p["q_rope"][0, 0] @ p["q_rope"][0, 0]) / math.sqrt(dn + dr)
    V = p["rows"][:, :dl] @ p["w_uv"][0].T
    wts = np.ones(L)
    wts[ts] = math.exp(sstar)
    assert_close(o[0], (wts @ V) / wts.sum())
    assert abs(lse[0] - math.log(wts.sum())) < 1e-13


def test_common_score_shift():
    rng = np.random.default_rng(16)
    p = rand_problem(rng, B=2, H=3, L=33)
    o0, lse0, _ = run(p)
    dn, dr, dl, dv = p["dims"]
    delta = rng.standard_normal(dr)
    p["rows"][:, dl:] += delta  # k_R of every token moves by the same vector
    o1, lse1, _ = run(p)
    assert_close(o1, o0, 1e-11)
    shift = (p["q_rope"] @ delta).reshape(-1) / math.sqrt(dn + dr)
    assert np.max(np.abs((lse1 - lse0) - shift)) < 1e-11


def test_token_and_head_permutation():
    rng = np.random.default_rng(17)
    p = rand_problem(rng, B=1, H=5, L=40)
    o0, lse0, _ = run(p)
    q = dict(p)
    q["rows"] = p["rows"][rng.permutation(40)]
    o1, lse1, _ = run(q)
    assert_close(o1, o0, 1e-12)
    assert_close(lse1, lse0, 1e-12)
    perm = rng.permutation(5)
    r = dict(p)
    for k in ("q_nope", "q_rope"):
        r[k] = p[k][:, perm]
    for k in ("w_uk", "w_uv"):
        r[k] = p[k][perm]
    o2, lse2, _ = run(r)
    assert_close(o2, o0[perm], 0)
    assert_close(lse2, lse0[perm], 0)


@pytest.mark.parametrize("cuts", [(0, 13, 40, 61), (0, 0, 61, 61), (0, 1, 2, 30, 61)])
def test_split_and_merge_equals_whole(cuts):
    rng = np.random.default_rng(18)
    p = rand_problem(rng, B=2, H=3, L=61)
    o0, lse0, u0 = run(p, want_u=True)
    S = len(cuts) - 1
    dl = p["dims"][2]
    u_part = np.zeros((2, S, 3, dl))
    lse_part = np.zeros((2, S, 3))
    for s in range(S):
        _, l_s, u_s = run(p, want_u=True, t_begin=[cuts[s]] * 2, t_end=[cuts[s + 1]] * 2)
        u_part[:, s] = u_s.reshape(2, 3, dl)
        lse_part[:, s] = l_s.reshape(2, 3)
    u, lse = oracle.combine(u_part, lse_part)
    assert_close(u.reshape(-1, dl), u0, 1e-12)
    assert_close(lse.reshape(-1), lse0, 1e-12)
    o = oracle.up_proj(u, p["w_uv"], "f64")
    assert_close(o.reshape(6, -1), o0, 1e-12)


def test_empty_sequences():
    rng = np.random.default_rng(19)
    p = rand_problem(rng, B=3, H=2, L=8, lens=[0, 8, 0])
    o, lse, u = run(p, want_u=True)
    assert np.all(o[[0, 1, 4, 5]] == 0) and np.all(np.isneginf(lse[[0, 1, 4, 5]]))
    assert np.all(np.isfinite(o)) and np.all(u[[0, 1]] == 0)
    u_part = np.zeros((1, 2, 1, 4))
    lse_part = np.full((1, 2, 1), -np.inf)
    uu, ll = oracle.combine(u_part, lse_part)
    assert np.all(uu == 0) and np.isneginf(ll).all()


def test_linear_in_w_uv():
    rng = np.random.default_rng(20)
    p = rand_problem(rng)
    w2 = rng.standard_normal(p["w_uv"].shape)
    o1, _, _ = run(p)
    q = dict(p, w_uv=w2)
    o2, _, _ = run(q)
    r = dict(p, w_uv=p["w_uv"] + w2)
    o3, _, _ = run(r)
    assert_close(o3, o1 + o2, 1e-12)


def test_absorb_and_up_proj_calls():
    rng = np.random.default_rng(21)
    p = rand_problem(rng, B=2, H=3, L=5)
    qa = oracle.absorb_q(p["q_nope"], p["q_rope"], "f64", p["w_uk"], "f64")
    for b in range(2):
        for h in range(3):
            assert_close(qa[b, h, :32], p["q_nope"][b, h] @ p["w_uk"][h])
            assert np.array_equal(qa[b, h, 32:], p["q_rope"][b, h])
    u = rng.standard_normal((2, 3, 32))
    o = oracle.up_proj(u, p["w_uv"], "f64")
    assert_close(o, np.einsum("hvc,bhc->bhv", p["w_uv"], u))


def test_absorb_q_and_up_proj_outputs_reproduce_the_naive_decode():
    """oracle.absorb_q's output, taken as the query of attention straight over
    the 576-wide cached rows [c_KV | k_R], and oracle.up_proj applied to the
    weighted latent sum, give the naive decode that rebuilds each head's keys
    and values (itself pinned to library SDPA above): absorbing W_UK into the
    query and applying W_UV after the sum is exact algebra ([V2] §2.3, §4.1),
    so they agree to rounding.  Widths differ (d_nope != d_latent != d_v) so
    a transposed weight index reads other elements."""
    rng = np.random.default_rng(23)
    B, H, L = 2, 5, 37
    p = rand_problem(rng, B=B, H=H, L=L, dn=24, dr=8, dl=40, dv=12)
    o_ref, lse_ref, u_ref = run(p, want_u=True)
    qa = oracle.absorb_q(p["q_nope"], p["q_rope"], "f64", p["w_uk"], "f64")
    dn, dr, dl, dv = p["dims"]
    assert qa.shape == (B, H, dl + dr)
    u = np.zeros((B, H, dl))
    lse = np.zeros((B, H))
    for b in range(B):
        rows = p["rows"][b * L:(b + 1) * L]
        s = (rows @ qa[b].T) / math.sqrt(dn + dr)  # [L, H]
        m = s.max(axis=0)
        w = np.exp(s - m)
        u[b] = (w.T @ rows[:, :dl]) / w.sum(axis=0)[:, None]
        lse[b] = m + np.log(w.sum(axis=0))
    assert_close(u.reshape(-1, dl), u_ref)
    assert_close(lse.reshape(-1), lse_ref)
    assert_close(oracle.up_proj(u, p["w_uv"], "f64").reshape(-1, dv), o_ref)


def test_default_scale_is_one_over_sqrt_nope_plus_rope():
    rng = np.random.default_rng(22)
    p = rand_problem(rng)
    o0, l0, _ = run(p)
    o1, l1, _ = run(p, scale=1 / math.sqrt(16 + 8))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    o2, _, _ = run(p, scale=1 / math.sqrt(32 + 8))
    assert np.max(np.abs(o2 - o0)) > 1e-6


def _small(wl_name, **kw):
    wl = synth.workload(wl_name).with_(**kw)
    return wl


def test_paged_equals_contiguous_and_poison_is_unread():
    wl_c = _small("dsv2_b32_l2k", batch=3, heads=4, seq_len=None, len_range=(1, 200),
                  seed=99)
    wl_p = wl_c.with_(page_size=64)
    lens = [200, 65, 3]
    ic = synth.make_inputs(wl_c, lengths=lens, seq_stride=256)  # NaN past each length
    ip = synth.make_inputs(wl_p, lengths=lens)  # NaN in each last page's tail
    assert np.isnan(oracle.decode_array(ic.rows, "bf16")).any()
    assert np.isnan(oracle.decode_array(ip.rows, "bf16")).any()
    oc, lc, _ = oracle.decode_inputs(ic)
    op, lp, _ = oracle.decode_inputs(ip)
    assert np.all(np.isfinite(oc)) and np.all(np.isfinite(lc))
    assert np.array_equal(oc, op) and np.array_equal(lc, lp)


def test_fp8_rows_are_decoded_codes_times_row_scale():
    wl = _small("fp8_b1_l128k", batch=2, heads=4, seq_len=70, seed=7)
    inp = synth.make_inputs(wl)
    o8, l8, _ = oracle.decode_inputs(inp)
    rows = oracle.decode_array(inp.rows, "fp8") * inp.row_scale.astype(np.float64)[:, None]
    o64, l64, _ = oracle.decode(inp.q_nope, inp.q_rope, "bf16", inp.w_uk, inp.w_uv, "bf16",
                                rows, "f64", inp.seq_lens, seq_stride=inp.seq_stride)
    assert np.array_equal(o8, o64) and np.array_equal(l8, l64)
