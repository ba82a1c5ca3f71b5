"""Pins of the oracle's FP8 (E4M3) encoding against a library implementation of the
same format, the format's own fixed points, and the closed-form footprint at b = 1
("PagedAttention and Virtual Memory Management", section 1)."""

import math

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

ALL = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_decode_equals_library_on_all_codes():
    a, b = oracle.fp8_to_f64(ALL), _torch_decode(ALL)
    nan = np.isnan(b)
    assert np.array_equal(np.isnan(a), nan) and nan.sum() == 2          # 0x7F, 0xFF
    assert np.array_equal(a[~nan], b[~nan])
    assert oracle.fp8_to_f64([0x7E])[0] == 448.0 and oracle.fp8_to_f64([0x01])[0] == 2.0 ** -9
    assert oracle.fp8_to_f64([0x08])[0] == 2.0 ** -6 and oracle.fp8_to_f64([0x38])[0] == 1.0


def test_encode_inverts_decode():
    v = oracle.fp8_to_f64(ALL)
    fin = ~np.isnan(v)
    assert np.array_equal(oracle.encode_fp8(v[fin]), ALL[fin])


def test_encode_equals_library_rounding_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 1e-2, 0.1, 1.0, 10.0, 100.0)])
    x = x[np.abs(x) < 440].astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_fp8(x), want)


def test_midpoints_round_to_the_even_code():
    v = oracle.fp8_to_f64(ALL[:0x7F])          # non-negative finite codes, ascending
    for c in range(0x7E):
        lo, hi = v[c], v[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.encode_fp8([mid])[0] == even, hex(c)
        assert oracle.encode_fp8([math.nextafter(mid, 0)])[0] == c
        assert oracle.encode_fp8([math.nextafter(mid, math.inf)])[0] == c + 1
        assert oracle.encode_fp8([-mid])[0] == 0x80 | even


def test_saturation_and_nan():
    enc = oracle.encode_fp8
    assert list(enc([448.0, 460.0, 464.0, 1e6, math.inf])) == [0x7E] * 5
    assert list(enc([-448.0, -1e6, -math.inf])) == [0xFE] * 3
    assert enc([math.nan])[0] == 0x7F and enc([-math.nan])[0] == 0xFF
    assert enc([0.0])[0] == 0x00 and enc([-0.0])[0] == 0x80
    assert enc([2.0 ** -10])[0] == 0x00                  # half the smallest subnormal: tie to 0
    assert enc([1.5 * 2.0 ** -10])[0] == 0x01


def test_quantize_rows_from_16_bit():
    bits = np.array([0x3C00, 0x3C40, 0xBC00, 0x7C00], dtype=np.uint16)   # f16: 1, 1.0625, -1, inf
    assert list(oracle.quantize_fp8(bits, "f16")) == [0x38, 0x38, 0xB8, 0x7E]
    bits = np.array([0x3F80, 0x4400], dtype=np.uint16)                    # bf16: 1, 512
    assert list(oracle.quantize_fp8(bits, "bf16")) == [0x38, 0x7E]


def test_footprint_at_one_byte():
    # Llama-3-8B: 2 * 32 layers * 8 heads * 128 * b; b = 1 halves the 131,072 B of b = 2
    assert oracle.kv_bytes_per_token(32, 8, 128, 1) == 65536
    assert oracle.kv_pool_bytes(32, 8, 128, 1, 1000, 16) == 65536 * 16000


def test_fp8_attention_reads_decoded_values():
    rng = np.random.default_rng(1)
    codes_k = oracle.encode_fp8(rng.standard_normal((3, 16, 2, 8)))
    codes_v = oracle.encode_fp8(rng.standard_normal((3, 16, 2, 8)))
    q = (rng.standard_normal((4, 8)) * 8).round().astype(np.float64)
    qbits = q.astype(np.float16).view(np.uint16)
    table, L = [2, 0, 1], 40
    got = oracle.paged_decode_seq(qbits, codes_k, codes_v, table, L, 0.3, 16, "fp8", q_dtype="f16")
    kc = oracle.fp8_to_f64(oracle.gather(codes_k, table, L, 16))
    vc = oracle.fp8_to_f64(oracle.gather(codes_v, table, L, 16))
    want = oracle.attention_contiguous(q, kc, vc, 0.3)
    assert np.allclose(got, want, rtol=0, atol=1e-13)
