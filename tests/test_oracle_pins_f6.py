"""Pins of the oracle's FP6 operand encoding (not a step of the pages' method: an exact re-encoding
of the int4 codes for the FP6 matrix instructions).

- The E3M2 decoder against the landmark values of the OCP Microscaling format's definition
  (exponent bias 3: largest normal 28, smallest normal 0.25, largest subnormal 0.1875, smallest
  subnormal 0.0625, 1.0 = exponent field 3 with a zero mantissa).
- The encoder: each integer in [-8, 7] gets a distinct code whose decoded value is that integer;
  sign symmetry for the magnitudes both signs share.
- The operand layout against bytes derived by hand from its definition (first codes of a row, the
  field that straddles the head / tail split, the tail, a later stage and group, the zero pad row).
- Round trip and a brute-force dot product: decoding two encoded operands and multiplying in fp64
  gives the integer GEMM of the codes.
"""
import numpy as np
import pytest

import oracle


def test_e3m2_landmarks():
    assert oracle.e3m2_value(0b0_111_11) == 28.0
    assert oracle.e3m2_value(0b1_111_11) == -28.0
    assert oracle.e3m2_value(0b0_001_00) == 0.25
    assert oracle.e3m2_value(0b0_000_11) == 0.1875
    assert oracle.e3m2_value(0b0_000_01) == 0.0625
    assert oracle.e3m2_value(0b0_011_00) == 1.0
    assert oracle.e3m2_value(0b0_000_00) == 0.0
    assert oracle.e3m2_value(0b0_100_10) == 3.0  # 2^(4-3) * (1 + 2/4)


def test_e3m2_encode_int4_grid():
    codes = [oracle.e3m2_encode(v) for v in range(-8, 8)]
    assert len(set(codes)) == 16
    for v, c in zip(range(-8, 8), codes):
        assert oracle.e3m2_value(c) == v
        assert 0 <= c < 64
    for v in range(1, 8):
        assert oracle.e3m2_encode(-v) == oracle.e3m2_encode(v) | 0x20
    assert oracle.e3m2_encode(0) == 0
    with pytest.raises(ValueError):
        oracle.e3m2_encode(8)


def test_f6_layout_hand_bytes():
    rows, K = 3, 256
    q = np.zeros((rows, K), np.int8)
    q[0, 0:4] = [1, 2, 3, -1]  # E3M2 0x0C, 0x10, 0x12, 0x2C
    q[0, 21] = 7               # 0x17 at bits 126..131: two bits in head byte 15, four in tail byte 0
    q[1, 22] = 1               # 0x0C at bits 132..137 = tail bits 4..9
    q[2, 128 + 32] = -8        # stage 1, group 1, first field: 0x38
    buf = oracle.f6_operand(q)
    R2 = 4
    assert buf.size == R2 * K * 3 // 4 == oracle.f6_bytes(rows, K)
    stage = buf.reshape(K // 128, R2 * 96)
    head = stage[:, :R2 * 64].reshape(K // 128, R2, 4, 16)   # [stage][row][group][16 bytes]
    tail = stage[:, R2 * 64:].reshape(K // 128, 4, R2, 8)    # [stage][group][row][8 bytes]
    # bits 0..5 = 0x0C, 6..11 = 0x10, 12..17 = 0x12, 18..23 = 0x2C
    assert list(head[0, 0, 0, :3]) == [0x0C, 0x24, 0xB1]
    assert head[0, 0, 0, 15] == 0xC0 and tail[0, 0, 0, 0] == 0x05
    assert list(tail[0, 0, 1, :2]) == [0xC0, 0x00]
    assert head[1, 2, 1, 0] == 0x38 and tail[1, 1, 2].sum() == 0
    assert buf[384 + 64 * 2 + 16] == 0x38    # stage 0 is 4 * 96 = 384 bytes; head (2, 1) at 128 + 16
    assert not head[:, 3].any() and not tail[:, :, 3].any()  # pad row
    assert np.count_nonzero(buf) == 7


@pytest.mark.parametrize("rows,K", [(1, 128), (5, 256), (16, 384)])
def test_f6_round_trip_and_dot(rows, K):
    rng = np.random.default_rng(rows * 1000 + K)
    q = rng.integers(-8, 8, (rows, K)).astype(np.int8)
    p = rng.integers(-8, 8, (7, K)).astype(np.int8)
    bq, bp = oracle.f6_operand(q), oracle.f6_operand(p)
    assert (oracle.f6_codes(bq, rows, K) == q).all()
    dec = np.vectorize(oracle.e3m2_value)

    def values(buf, n):
        R2 = (n + 1) // 2 * 2
        stage = buf.reshape(K // 128, R2 * 96)
        head = stage[:, :R2 * 64].reshape(K // 128, R2, 4, 16)
        tail = stage[:, R2 * 64:].reshape(K // 128, 4, R2, 8)
        out = np.zeros((n, K))
        for r in range(n):
            for sg in range(K // 32):
                st, g = divmod(sg, 4)
                bits = int.from_bytes(bytes(head[st, r, g]) + bytes(tail[st, g, r]), "little")
                out[r, 32 * sg:32 * sg + 32] = dec([(bits >> (6 * i)) & 63 for i in range(32)])
        return out

    y = values(bq, rows) @ values(bp, 7).T
    brute = np.array([[sum(int(q[m, k]) * int(p[n, k]) for k in range(K)) for n in range(7)]
                      for m in range(rows)])
    assert (y == brute).all()
    assert (oracle.int_gemm(q, p) == brute).all()
