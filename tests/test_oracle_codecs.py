"""The oracle's storage-format decoders against the format definitions and torch."""
import math

import numpy as np
import torch

from oracle import attention as A


def test_fp16_known_values():
    cases = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x3555: 0.333251953125, 0x8000: -0.0}
    bits = np.array(list(cases), dtype=np.uint16)
    got = A.decode_fp16(bits)
    assert list(got) == list(cases.values())
    assert math.copysign(1.0, got[-1]) == -1.0


def test_fp16_all_codes_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    got = A.decode_fp16(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_bf16_known_values():
    cases = {0x3F80: 1.0, 0xC040: -3.0, 0x0001: 2.0 ** -133,
             0x7F7F: float(np.float32(3.3895313892515355e38)), 0x3EAB: 0.333984375}
    got = A.decode_bf16(np.array(list(cases), dtype=np.uint16))
    assert list(got) == list(cases.values())


def test_bf16_all_codes_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = A.decode_bf16(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_known_values():
    # OCP 8-bit FP, E4M3: bias 7, max normal 0x7E = 1.75 * 2^8 = 448, min normal
    # 0x08 = 2^-6, min subnormal 0x01 = 2^-9, NaN at S.1111.111, no infinities.
    cases = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x40: 2.0,
             0x3C: 1.5, 0x77: 240.0 * 1.0 + 0.0}
    got = A.decode_e4m3(np.array(list(cases), dtype=np.uint8))
    assert list(got) == list(cases.values())
    assert np.isnan(A.decode_e4m3(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    assert math.copysign(1.0, A.decode_e4m3(np.array([0x80], dtype=np.uint8))[0]) == -1.0


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = A.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # Every finite code is distinct apart from +0 / -0.
    finite = got[ok]
    assert len(np.unique(finite)) == len(finite) - 1
