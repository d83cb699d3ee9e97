"""Pins for the oracle's tiled 2-bit format reader and its quantizer.

* a hand-derived worked example (tests/golden/q2_tile_layout.txt) pins every
  index of the layout (lane, word, nibble, record order, scale position);
* the dequantize -> quantize -> dequantize round trip on exact grid values is
  bit exact, the check the pages describe for Q2_0 ("32GB Mac mini ...",
  section 四, second validation layer);
* sizes at the workload shapes.
"""
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q2_tile_layout.txt")


def _load_golden():
    R = K = None
    byts, scales, expects = [], [], []
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "matrix":
            R, K = int(f[1]), int(f[2])
        elif f[0] == "byte":
            byts.append((int(f[1]), int(f[2], 16)))
        elif f[0] == "scale_at":
            scales.append((int(f[1]), float(f[2])))
        elif f[0] == "expect":
            expects.append((int(f[1]), int(f[2]), float(f[3])))
    return R, K, byts, scales, expects


def test_golden_tile_layout():
    R, K, byts, scales, expects = _load_golden()
    buf = np.zeros(O.matrix_nbytes(R, K), dtype=np.uint8)
    for off, v in byts:
        buf[off] = v
    for off, v in scales:
        buf[off:off + 2] = np.frombuffer(np.float16(v).tobytes(), dtype=np.uint8)
    W = O.dequantize(*O.decode_matrix(buf, 0, R, K))
    assert len(expects) >= 15
    for r, c, v in expects:
        assert W[r, c] == v, (r, c, W[r, c], v)


def test_golden_encode_matches_bytes():
    """The packer writes exactly the hand-derived bytes for the same codes."""
    R, K, byts, scales, _ = _load_golden()
    buf = np.zeros(O.matrix_nbytes(R, K), dtype=np.uint8)
    for off, v in byts:
        buf[off] = v
    for off, v in scales:
        buf[off:off + 2] = np.frombuffer(np.float16(v).tobytes(), dtype=np.uint8)
    codes, sc = O.decode_matrix(buf, 0, R, K)
    assert np.array_equal(O.encode_matrix(codes, sc), buf)


@pytest.mark.parametrize("R,K", [(16, 256), (48, 512), (256, 1024), (1024, 256)])
def test_encode_decode_roundtrip(R, K):
    rng = np.random.default_rng(R * 7 + K)
    codes = rng.integers(0, 4, size=(R, K), dtype=np.uint8)
    sc = rng.uniform(-3, 3, size=(R, K // 32)).astype(np.float16)
    buf = O.encode_matrix(codes, sc)
    assert buf.size == O.matrix_nbytes(R, K)
    c2, s2 = O.decode_matrix(buf, 0, R, K)
    assert np.array_equal(c2, codes)
    assert np.array_equal(s2.view(np.uint16), sc.view(np.uint16))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dequant_quant_roundtrip_bit_exact(seed):
    rng = np.random.default_rng(seed)
    R, K = 64, 512
    codes = rng.integers(0, 4, size=(R, K), dtype=np.uint8)
    d = rng.uniform(0.01, 0.05, size=(R, K // 32)).astype(np.float16)
    # blocks that never use code 0 or code 3, and all-zero blocks
    codes[0, :32] = rng.integers(1, 3, size=32)
    codes[1, 32:64] = 1
    codes[2, :32] = rng.integers(1, 4, size=32)
    W = O.dequantize(codes, d)
    q2, d2 = O.quantize_q2(W)
    W2 = O.dequantize(q2, d2)
    assert np.array_equal(W2.view(np.uint64), W.view(np.uint64))
    # the all-zero block gets d = 0, q = 1
    assert d2[1, 1] == 0 and np.all(q2[1, 32:64] == 1)
    # through the byte format too
    W3 = O.dequantize(*O.decode_matrix(O.encode_matrix(q2, d2), 0, R, K))
    assert np.array_equal(W3, W)


def test_dequant_codebook_values():
    """Affine codebook with bias -1: codes 0,1,2,3 -> -d, 0, d, 2d."""
    codes = np.tile(np.arange(4, dtype=np.uint8), (16, 64))
    d = np.full((16, 8), 0.25, dtype=np.float16)
    W = O.dequantize(codes, d)
    assert np.array_equal(W[0, :4], [-0.25, 0.0, 0.25, 0.5])


def test_workload_sizes():
    # 512-expert layer, hidden 3072, intermediate 768: 2,211,840 B per expert
    lay = O.expert_layout(3072, 768)
    assert lay["nbytes"] == 2_211_840 and lay["stride"] == 2_211_840
    assert lay["up"] == 737_280 and lay["down"] == 2 * 737_280
    # 64-expert layer, hidden 1024, intermediate 256
    assert O.expert_layout(1024, 256)["nbytes"] == 245_760
    with pytest.raises(ValueError):
        O.matrix_nbytes(16, 100)
