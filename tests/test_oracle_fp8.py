"""Pins of the FP8 oracle (CPU only): e4m3fn rounding against the OCP
landmarks and torch's float8_e4m3fn cast (a library routine), and properties
that the per-token quantizer must have whatever its implementation."""
import os

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3(x32):
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_ocp_landmarks():
    for line in open(os.path.join(GOLDEN, "e4m3_landmarks.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        val, code = line.split()
        v = float(val)
        r = oracle.e4m3_round(np.array([v], np.float32))
        assert r[0] == v or (v == 0 and r[0] == 0)
        assert oracle.e4m3_encode(r)[0] == int(code, 16), line
        assert oracle.e4m3_decode(np.array([int(code, 16)], np.uint8))[0] == v


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_round(vals.astype(np.float32))), codes)
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_rounding_matches_torch_cast_including_ties():
    finite = np.sort(np.unique(oracle.e4m3_decode(
        np.array([c for c in range(128) if c != 0x7F], np.uint8))))
    mids = (finite[:-1] + finite[1:]) / 2                   # exact ties
    rng = np.random.default_rng(0)
    rand = rng.uniform(-448, 448, 200000)
    small = rng.uniform(-0.05, 0.05, 50000)
    x = np.concatenate([finite, -finite, mids, -mids, np.nextafter(mids, 0),
                        np.nextafter(mids, 1000), rand, small]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ours = oracle.e4m3_encode(oracle.e4m3_round(x))
    assert np.array_equal(ours, _torch_e4m3(x))


def test_saturation_reading():
    r = oracle.e4m3_round(np.array([449.0, 463.9, 1e6, -5000.0], np.float32))
    assert list(r) == [448.0, 448.0, 448.0, -448.0]


def test_quantizer_properties():
    w = synth.WORKLOADS["tiny"].replace(outlier_frac=0.05)
    q, k, v, _ = synth.make_qkv(w, seed=1)
    v = v.clone()
    v[0, 3, 1] = 0.0                                        # an all-zero head vector
    pos = synth.positions(w)
    q8, k8, v8, sq, sk, sv = oracle.quant_rope_fp8(q, k, v, pos)
    for x8, s in ((q8, sq), (k8, sk), (v8, sv)):
        vals = oracle.e4m3_decode(x8)
        amax = np.abs(vals).max(-1)                         # [B, S, H]
        nz = np.transpose(s, (0, 2, 1)) != 1.0
        # the largest element of every non-zero vector lands exactly on 448
        assert np.all(amax[nz] == 448.0)
        assert x8.dtype == np.uint8 and s.dtype == np.float32
    assert sv[0, 1, 3] == 1.0 and np.all(v8[0, 3, 1] == 0)
    # dequantization error is at most half an e4m3 spacing of x/scale
    qr = oracle.apply_rope(q, pos).numpy()
    deq = oracle.dequantize(q8, sq).numpy()
    y = qr / np.transpose(sq, (0, 2, 1))[..., None]
    _, e = np.frexp(np.abs(y))
    half_ulp = np.ldexp(1.0, np.maximum(e - 1, -6) - 4)
    err = np.abs(deq - qr) / np.transpose(sq, (0, 2, 1))[..., None]
    assert np.all(err <= half_ulp * (1 + 1e-6) + 1e-6)


def test_fp8_attention_on_exact_inputs_is_plain_attention():
    # Inputs that are already e4m3 values with amax 448 quantize to scale 1
    # and themselves, so the FP8 reference must equal plain attention.
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7E, size=(1, 24, 2, 64)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    codes[..., 5] = 0x7E
    x = torch.from_numpy(oracle.e4m3_decode(codes)).to(torch.float32)
    q8, k8, v8, sq, sk, sv = oracle.quant_rope_fp8(x, x * 0.5, x, None)
    assert np.array_equal(q8, codes) and np.all(sq == 1.0) and np.all(sk == 0.5)
    o, _ = oracle.fp8_attention(q8, k8, v8, sq, sk, sv)
    ref, _ = oracle.attention(x, x * 0.5, x)
    assert torch.allclose(o, ref, atol=1e-12)
