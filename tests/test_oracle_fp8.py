"""Pins of the FP8 E4M3 cache oracle (oracle/fp8.py), CPU only:

- every one of the 256 codes against torch's float8_e4m3fn conversion (a
  library decoder written independently of this one), NaN codes included;
- hand values from the format definition (1.0, the largest finite, the
  smallest subnormal, negative zero);
- attention over byte caches = attention over the caches torch decodes, with
  the scales applied, bit for bit in float64;
- the one-row helper against the full oracle;
- planted decoder mistakes (exponent bias 8, no subnormals, sign dropped)
  each fail the library comparison.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as of
from workloads import build_attention, decode_queries


def test_all_codes_match_torch():
    codes = np.arange(256)
    ours = oracle.e4m3_decode(codes)
    theirs = torch.as_tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    np.testing.assert_array_equal(ours[ok], theirs[ok])
    np.testing.assert_array_equal(np.signbit(ours[ok]), np.signbit(theirs[ok]))
    assert int(np.isnan(ours).sum()) == 2  # S.1111.111 only


def test_hand_values():
    d = oracle.e4m3_decode
    assert d(0x38) == 1.0                     # exponent 7, mantissa 0
    assert d(0x7E) == 448.0                   # 2^8 * 1.75, the largest finite
    assert d(0x01) == 2.0 ** -9               # smallest subnormal: 1/8 * 2^-6
    assert d(0x08) == 2.0 ** -6               # smallest normal
    assert d(0xB8) == -1.0
    assert d(0x80) == 0.0 and np.signbit(d(0x80))


def _fp8_case(seed, lens, hq=4, hkv=2, d=16, ps=8):
    wl = build_attention("f8", seed, torch.float32, lens, decode_queries(lens), hq, hkv, d, d, ps)
    gen = torch.Generator().manual_seed(seed)
    k8 = torch.randint(0, 256, tuple(wl.tensors["k"].shape), generator=gen, dtype=torch.uint8)
    v8 = torch.randint(0, 256, tuple(wl.tensors["v"].shape), generator=gen, dtype=torch.uint8)
    # no NaN codes: finite caches
    k8[(k8 & 0x7F) == 0x7F] = 0x7E
    v8[(v8 & 0x7F) == 0x7F] = 0x7E
    return wl, k8, v8


def test_attention_equals_attention_on_decoded_caches():
    wl, k8, v8 = _fp8_case(5, [40, 9, 100])
    ks, vs = 0.03125, 0.0078125
    got, lse = oracle.paged_attention_fp8(wl.tensors["q"], k8, v8, wl.lens, wl.qseq, wl.qpos,
                                          wl.table, wl.page_size, wl.scale, True, ks, vs)
    kd = k8.view(torch.float8_e4m3fn).to(torch.float64) * ks
    vd = v8.view(torch.float8_e4m3fn).to(torch.float64) * vs
    want, lse2 = oracle.paged_attention(wl.tensors["q"], kd, vd, wl.lens, wl.qseq, wl.qpos,
                                        wl.table, wl.page_size, wl.scale, True)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(lse, lse2)


def test_one_row_helper_matches():
    wl, k8, v8 = _fp8_case(6, [70, 33])
    args = (wl.tensors["q"], k8, v8, wl.lens, wl.qseq, wl.qpos, wl.table, wl.page_size,
            wl.scale, True)
    full, _ = oracle.paged_attention_fp8(*args, 0.05, 0.02, window=20)
    for i in range(2):
        for h in (0, 3):
            row, _ = oracle.attention_one_fp8(*args, i, h, 0.05, 0.02, window=20)
            np.testing.assert_allclose(row, full[i, h], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("planted", [
    lambda c: np.where((c & 0x78) == 0, 0.0, np.ldexp(1.0 + (c & 7) / 8.0, ((c >> 3) & 15) - 8)),
    lambda c: np.ldexp(1.0 + (c & 7) / 8.0, ((c >> 3) & 15) - 7),
    lambda c: np.abs(oracle.e4m3_decode(c)),
])
def test_planted_decoder_mistakes_fail(planted):
    codes = np.arange(256)
    bad = planted(codes).astype(np.float64)
    theirs = torch.as_tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ok = ~np.isnan(theirs)
    assert not np.array_equal(bad[ok], theirs[ok])
