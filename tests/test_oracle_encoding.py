"""Pins of the oracle's element encodings against torch's own conversions."""

import numpy as np
import torch

from oracle import encoding


def _edge_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 1e-45, -1e-45, 1.17549435e-38, 3.4028235e38, -3.4028235e38,
            np.inf, -np.inf, 65504.0, 65520.0, 6.1e-5, 5.96e-8]
    x = np.array(vals, dtype=np.float32)
    # exact ties: low 16 bits == 0x8000 with even and odd kept parts
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000, 0x00008000, 0x00018000], dtype=np.uint32)
    near = np.array([0x3F807FFF, 0x3F808001, 0x3F80FFFF, 0x3F7FFFFF], dtype=np.uint32)
    return np.concatenate([x, ties.view(np.float32), near.view(np.float32)])


def test_bf16_round_nearest_even_matches_torch():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        _edge_f32(),
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    finite = ~np.isnan(x)
    ours = encoding.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours[finite], ref[finite])
    # NaN stays NaN (torch picks one quiet NaN; so do we)
    assert np.all(np.isnan(encoding.bf16_bits_to_f64(ours[~finite])))


def test_fp16_and_fp32_round_trip_match_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([_edge_f32(), rng.standard_normal(100_000).astype(np.float32)])
    x = x[~np.isnan(x)]
    h = encoding.encode(x, "f16")
    ref = torch.from_numpy(x.copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, ref)
    got = encoding.decode(h, "f16")
    assert np.array_equal(got, torch.from_numpy(ref.view(np.float16).copy()).double().numpy())
    f = encoding.encode(x, "f32")
    assert np.array_equal(encoding.decode(f, "f32"), x.astype(np.float64))


def test_bf16_decode_is_upper_half():
    rng = np.random.default_rng(9)
    b = rng.integers(0, 2**16, 10_000).astype(np.uint16)
    got = encoding.decode(b, "bf16")
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
