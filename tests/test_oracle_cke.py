"""Pins of the oracle's CKE split-half NVFP4 block ("Why 4-Bit Quantization Is
King", section 5): 64 weights in 36 bytes, four E4M3 subscales then 32 code
bytes, inside each 16-weight subblock the low nibbles of eight bytes are
weights 0-7 and the high nibbles weights 8-15, reconstructed by the NVFP4 rule
(E2M1 * E4M3) * scale2.

- A hand-built block (tests/golden/nvfp4_cke_block.json) whose 64 values are
  written out from the page's codebook: it fixes the lane order, the subscale
  order and the reconstruction, and the same bytes read in the adjacent-pair
  order give different values, so a mix-up of the two orders fails here.
- 36 bytes per 64 weights = 4.5 bits per weight, the page's figure.
- Against the separately pinned NVFP4 decoder: the same logical codes and
  subscales, packed split-half here and adjacent-pair there, dequantize to
  bit-identical values and give identical dot products.
"""
import json
import os

import numpy as np

import oracle

_GOLD = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_cke_block.json")


def _fixture():
    with open(_GOLD) as f:
        return json.load(f)


def _bits(v):
    return np.asarray(v, dtype=np.float32).view(np.uint32)


def test_golden_block_values():
    fx = _fixture()
    block = np.array(fx["block"], dtype=np.uint8)
    assert block.size == 36
    got = oracle.dequant_rows(oracle.NVFP4_CKE, block, None, fx["scale2"], 64, [0])[0]
    assert np.array_equal(_bits(got), _bits(fx["values"])), (got, fx["values"])


def test_golden_subscales_are_the_first_four_bytes():
    fx = _fixture()
    for j, v in enumerate(fx["subscale_values"]):
        assert oracle.e4m3fn(fx["block"][j]) == v


def test_golden_pack_and_unpack():
    fx = _fixture()
    codes = np.array(fx["codes"], dtype=np.uint8).reshape(1, 64)
    scales = np.array(fx["block"][:4], dtype=np.uint8).reshape(1, 4)
    assert np.array_equal(oracle.cke_pack(codes, scales).reshape(36), np.array(fx["block"], dtype=np.uint8))
    c, s = oracle.cke_unpack(np.array(fx["block"], dtype=np.uint8), 1, 64)
    assert np.array_equal(c, codes) and np.array_equal(s, scales)


def test_adjacent_pair_reading_of_the_same_bytes_differs():
    """The page's warning: interleaving instead of split-half order puts
    correct arithmetic on the wrong lanes. The fixture tells them apart."""
    fx = _fixture()
    block = np.array(fx["block"], dtype=np.uint8)
    as_adjacent = oracle.dequant_rows(oracle.NVFP4, block[4:].reshape(1, 32), block[:4].reshape(1, 4),
                                      fx["scale2"], 64, [0])[0]
    assert not np.array_equal(_bits(as_adjacent), _bits(fx["values"]))


def test_storage_is_four_and_a_half_bits_per_weight():
    rng = np.random.default_rng(0)
    n, k = 3, 256
    blocks = oracle.cke_pack(rng.integers(0, 16, (n, k)).astype(np.uint8),
                             rng.integers(0x18, 0x51, (n, k // 16)).astype(np.uint8))
    assert blocks.nbytes * 8 / (n * k) == 4.5


def _adjacent(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_matches_the_adjacent_pair_nvfp4_decoder():
    rng = np.random.default_rng(1)
    n, k = 5, 320
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    scales = rng.integers(0, 0x7F, (n, k // 16)).astype(np.uint8)  # every finite positive byte, zero included
    scale2 = float(np.float32(0.0123))
    cke = oracle.cke_pack(codes, scales)
    a = oracle.dequant_rows(oracle.NVFP4_CKE, cke, None, scale2, k, range(n))
    b = oracle.dequant_rows(oracle.NVFP4, _adjacent(codes), scales, scale2, k, range(n))
    assert np.array_equal(_bits(a), _bits(b))
    x = rng.standard_normal(k).astype(np.float32)
    ya, sa = oracle.gemv_rows(oracle.NVFP4_CKE, cke, None, scale2, k, x, range(n))
    yb, sb = oracle.gemv_rows(oracle.NVFP4, _adjacent(codes), scales, scale2, k, x, range(n))
    assert np.array_equal(ya, yb) and np.array_equal(sa, sb)


def test_pack_is_a_bijection_on_bytes():
    rng = np.random.default_rng(2)
    n, k = 4, 192
    raw = rng.integers(0, 256, (n, k // 64, 36)).astype(np.uint8)
    c, s = oracle.cke_unpack(raw, n, k)
    assert c.max() <= 15
    assert np.array_equal(oracle.cke_pack(c, s), raw)
