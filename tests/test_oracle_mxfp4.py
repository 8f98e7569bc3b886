"""Pins of the oracle's MXFP4 -> FP8 E4M3 conversion (CPU only).

The conversion is the online dequantisation of MXFP4 expert weights into an
FP8 working format ("Day-0 Inference Adaptation for Ultra-Large MoE Models on
Domestic GPUs", section "Handling Low-Precision Expert Weights: Online
Conversion and Workspace Reuse"; "Day-0 Adaptation for Trillion-Parameter MoE
Models", section V). Each pin is independent of the oracle's code: the OCP
element table, a brute-force nearest-code search in exact integer arithmetic
over every E4M3 code, torch's float8_e4m3fn cast inside the finite range, a
hand-worked golden file, and the slot semantics of the expert gather.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_fp8_example.json")

# OCP MX v1.0, FP4 E2M1 element values of codes 0..7 (codes 8..15: negated)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _pack(codes):
    """Element codes [rows, cols] -> packed bytes [rows, cols/2], element 2i in
    the low nibble of byte i."""
    codes = np.asarray(codes, np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _e4m3_candidates():
    """(code, value * 2^SHIFT as a Python int, sign) for every finite E4M3 code
    from its bit fields: bias 7, subnormals m/8 * 2^-6, S.1111.111 is NaN."""
    out = []
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        # value = (8 + m) * 2^(e - 10) for normals, m * 2^(-9) for subnormals
        num, exp = ((8 + m), e - 10) if e > 0 else (m, -9)
        out.append((code, num, exp, s))
    return out


SHIFT = 400
CANDS = [(c, (n << (exp + SHIFT)), s) for c, n, exp, s in _e4m3_candidates()]
POS = [(c, v) for c, v, s in CANDS if s == 0]
MAXV = max(v for _, v in POS)


def _nearest_e4m3(num, exp, negative):
    """E4M3 code nearest to num * 2^exp (exact integers): ties to the code with
    an even mantissa; values beyond 448 saturate to 448."""
    v = num << (exp + SHIFT) if exp + SHIFT >= 0 else num >> -(exp + SHIFT)
    assert exp + SHIFT >= 0
    sign = 0x80 if negative else 0
    if v >= MAXV:
        return sign | 0x7E
    best = None
    for c, cv in POS:
        d = abs(cv - v)
        key = (d, c & 1)  # nearest, then even mantissa
        if best is None or key < best[0]:
            best = (key, c)
    return sign | best[1]


def test_e2m1_codes_are_the_ocp_values():
    """Codes 0..15 at scale 2^0 decode (through torch's E4M3 reading of the
    output) to the OCP E2M1 table and its negation."""
    codes = np.tile(np.arange(16, dtype=np.uint8), 2).reshape(1, 32)
    fp8 = O.mxfp4_to_fp8(_pack(codes), np.array([[127]], np.uint8), 1, 32)
    vals = torch.from_numpy(fp8.reshape(-1)).view(torch.float8_e4m3fn).float().numpy()
    expect = E2M1_TABLE + [-x for x in E2M1_TABLE]
    np.testing.assert_array_equal(vals[:16], np.array(expect, np.float32))
    assert np.signbit(vals[8]) and not np.signbit(vals[0])


@pytest.mark.parametrize("exp_offset", [0, -20, 9])
def test_every_code_and_scale_against_brute_force(exp_offset):
    """All 16 element codes x all 256 scale bytes: the nearest E4M3 code by an
    exhaustive search in exact integer arithmetic."""
    rows = 256
    codes = np.tile(np.repeat(np.arange(16, dtype=np.uint8), 2), (rows, 1))  # [256, 32]
    scales = np.arange(256, dtype=np.uint8).reshape(rows, 1)
    got = O.mxfp4_to_fp8(_pack(codes), scales, rows, 32, exp_offset)
    # element value = mag2 / 2 with mag2 in {0, 1, 2, 3, 4, 6, 8, 12}
    mag2 = [0, 1, 2, 3, 4, 6, 8, 12]
    for x in range(256):
        for code in range(16):
            g = int(got[x, 2 * code])
            assert g == int(got[x, 2 * code + 1])
            neg = code >= 8
            if x == 255:
                assert g == (0xFF if neg else 0x7F), (x, code)
                continue
            want = _nearest_e4m3(mag2[code & 7], x - 127 + exp_offset - 1, neg)
            assert g == want, (x, code, exp_offset, hex(g), hex(want))


def test_torch_float8_cast_agrees_inside_the_finite_range():
    """Random blocks whose values stay below 464 (where torch's cast to
    float8_e4m3fn also rounds to a finite code): the same bit patterns."""
    rng = np.random.default_rng(5)
    rows, cols = 64, 256
    codes = rng.integers(0, 16, (rows, cols), dtype=np.uint8)
    scales = rng.integers(100, 134, (rows, cols // 32), dtype=np.uint8)  # 6 * 2^6 = 384 at most
    got = O.mxfp4_to_fp8(_pack(codes), scales, rows, cols)
    vals = np.array(E2M1_TABLE + [-x for x in E2M1_TABLE])[codes] * \
        np.exp2(np.repeat(scales.astype(np.float64) - 127, 32, axis=1))
    want = torch.from_numpy(vals).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, want)


def test_golden_hand_worked_blocks():
    doc = json.load(open(GOLDEN))
    for case in doc["cases"]:
        cols = case["cols"]
        packed = np.frombuffer(bytes.fromhex(case["packed_hex"]), np.uint8).reshape(1, cols // 2)
        scales = np.array(case["scales"], np.uint8).reshape(1, cols // 32)
        got = O.mxfp4_to_fp8(packed, scales, 1, cols, case["exp_offset"])
        want = np.frombuffer(bytes.fromhex(case["fp8_hex"]), np.uint8)
        np.testing.assert_array_equal(got.reshape(-1), want, err_msg=case["note"])


def test_expert_slots_follow_the_router_ids():
    """Slot s holds expert ids[s] converted on its own; an id outside the pool
    leaves its slot as it was; repeated ids fill several slots alike."""
    rng = np.random.default_rng(7)
    E, rows, cols = 5, 3, 64
    packed = rng.integers(0, 256, (E, rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(110, 140, (E, rows, cols // 32), dtype=np.uint8)
    ids = np.array([3, -1, 0, 3, 5], np.int32)
    out = np.full((ids.size, rows, cols), 0xAB, np.uint8)
    O.mxfp4_to_fp8_experts(packed, scales, E, rows, cols, ids, out=out)
    for s, e in enumerate(ids):
        if 0 <= e < E:
            np.testing.assert_array_equal(out[s], O.mxfp4_to_fp8(packed[e], scales[e], rows, cols))
        else:
            assert (out[s] == 0xAB).all()
    np.testing.assert_array_equal(out[0], out[3])


def test_bad_arguments_are_refused():
    with pytest.raises(ValueError):
        O.mxfp4_to_fp8(np.zeros(16, np.uint8), np.zeros(1, np.uint8), 1, 33)  # cols % 32
    with pytest.raises(ValueError):
        O.mxfp4_to_fp8(np.zeros(16, np.uint8), np.zeros(1, np.uint8), 1, 32, 2000)
