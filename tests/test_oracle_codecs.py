"""Pins the oracle's element decoders (exhaustively) and the input generator's
encoders against torch's own bfloat16 / float8_e4m3fn conversions and the OCP
E4M3 definition."""

import numpy as np
import torch

import oracle
import synth


def test_bf16_decode_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_array(codes, "bf16")
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode_array(codes, "fp8")
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 only: no infinities in E4M3 (OCP spec)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_spec_values():
    d = oracle.lib().oracle_decode_e4m3
    assert d(0x7E) == 448.0  # largest finite
    assert d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6  # smallest normal
    assert d(0x01) == 2.0 ** -9  # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9
    assert d(0x38) == 1.0
    assert d(0x39) == 1.125
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))


def test_bf16_decode_spec_values():
    d = oracle.lib().oracle_decode_bf16
    assert d(0x3F80) == 1.0
    assert d(0xC000) == -2.0
    assert d(0x7F7F) == (2 - 2.0 ** -7) * 2.0 ** 127  # largest finite
    assert d(0x0001) == 2.0 ** -133  # smallest subnormal
    assert np.isinf(d(0x7F80))


def test_generator_bf16_encoder_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact ties between two bf16 neighbours, both parities
    ties = (np.arange(1, 2000, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), -ties.view(np.float32)])
    got = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_generator_e4m3_quantizer_matches_torch_and_roundtrips():
    rng = np.random.default_rng(1)
    rows = rng.standard_normal((512, 576)).astype(np.float32)
    rows[3] = 0.0  # an all-zero row keeps a tiny positive scale
    rows[5, :10] = 1e-30
    codes, scale = synth.quantize_rows_e4m3(rows)
    assert scale.dtype == np.float32 and np.all(scale > 0)
    y = np.clip(rows / scale[:, None], -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # -0 and +0 are the same value
    both0 = (oracle.decode_array(codes, "fp8") == 0) & (oracle.decode_array(ref, "fp8") == 0)
    assert np.array_equal(np.where(both0, 0, codes), np.where(both0, 0, ref))
    # every finite code decodes and re-encodes to itself
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.decode_array(finite, "fp8").astype(np.float32)
    re, s = synth.quantize_rows_e4m3(np.concatenate([vals, [448.0]]).astype(np.float32)[None])
    assert s[0] == np.float32(1.0)
    z = vals == 0
    assert np.array_equal(re[0, :-1][~z], finite[~z])
    # the row maximum maps to 448 exactly
    amax_pos = np.argmax(np.abs(rows), axis=1)
    top = np.abs(oracle.decode_array(codes[np.arange(512), amax_pos], "fp8"))
    assert top[3] == 0 and np.all(np.delete(top, 3) == 448.0)
