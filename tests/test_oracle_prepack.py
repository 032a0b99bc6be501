"""Pins for the oracle's weight unpack and PB-v1 prepack (CPU only).

* nibble decode: exhaustive over all 256 byte values against the two's
  complement definition written out differently (sign bit test);
* PB-v1: bijection, round trip through the independently written inverse,
  single-nibble probes, and a *consumer* simulation: the bit operations a GEMM
  applies to a packed word must yield the logical values in k order;
* the F16 operand class reproduces the ExLlama word printed on the W4A16 page
  (golden fixture).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import w4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_nibble_decode_exhaustive():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    K = 512
    i4 = O.weight_values(b, K, "int4")[0]
    u4 = O.weight_values(b, K, "uint4")[0]
    b8 = O.weight_values(b, K, "uint4b8")[0]
    for byte in range(256):
        for half, code in ((0, byte & 15), (1, byte >> 4)):
            k = 2 * byte + half
            signed = -(code & 8) + (code & 7)        # two's complement by bit weights
            assert i4[k] == signed
            assert u4[k] == code
            assert b8[k] == code - 8


def _random_logical(N, K, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, (N, K // 2), dtype=np.uint8)


@pytest.mark.parametrize("operand", ["i8", "f16"])
def test_pb_v1_is_a_bijection(operand):
    N, K = 48, 384
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    word, shift = O.pb_v1_position(n.ravel(), k.ravel(), K, operand)
    assert word.min() == 0 and word.max() == N * K // 8 - 1
    assert set(np.unique(shift).tolist()) == {0, 4, 8, 12, 16, 20, 24, 28}
    flat = word * 8 + shift // 4
    assert np.unique(flat).size == N * K


@pytest.mark.parametrize("operand", ["i8", "f16"])
@pytest.mark.parametrize("shape", [(16, 128), (32, 256), (64, 1152), (272, 640)])
def test_pb_v1_round_trip(operand, shape):
    N, K = shape
    w = _random_logical(N, K, N * 7 + K)
    packed = O.prepack_B(w, N, K, operand)
    assert packed.dtype == np.uint8 and packed.size == N * K // 2
    assert np.array_equal(O.unprepack_B(packed, N, K, operand), w)


@pytest.mark.parametrize("operand", ["i8", "f16"])
def test_pb_v1_single_nibble_probes(operand):
    """Every one of the 2048 positions of a 16x128 block, one at a time."""
    N, K = 16, 128
    for n in range(N):
        for k in range(K):
            vals = np.zeros((N, K), dtype=np.uint8)
            vals[n, k] = 0xA
            w = (vals[:, 0::2] | (vals[:, 1::2] << 4)).astype(np.uint8)
            words = O.prepack_B(w, N, K, operand).view(np.uint32)
            nz = np.nonzero(words)[0]
            assert nz.size == 1
            d = int(nz[0])
            lane, kw = d // 4, d % 4
            assert lane % 16 == n and lane // 16 == k // 32 and kw == (k % 32) // 8
            p = [i for i in range(8) if (int(words[d]) >> (4 * i)) & 15][0]
            j = k % 8
            expect_p = (2 * j if j < 4 else 2 * (j - 4) + 1) if operand == "i8" else (j // 2 + 4 * (j % 2))
            assert p == expect_p


def _consumer_view_i8(words_lane):
    """What an int8/fp8 GEMM does with one lane's four words: keep the low
    nibbles of the four bytes (k 0..3 of the word) then the high nibbles
    (k 4..7).  Returns the 32 codes in the order they feed the MMA."""
    out = []
    for w in words_lane:
        lo = [((w >> (8 * b)) & 0xF) for b in range(4)]
        hi = [((w >> (8 * b + 4)) & 0xF) for b in range(4)]
        out += lo + hi
    return out


def _consumer_view_f16(words_lane):
    """What an fp16/bf16 GEMM does: (w >> 4i) & 0x000F000F gives the pair
    (k 2i, k 2i+1) in the low / high half-word."""
    out = []
    for w in words_lane:
        for i in range(4):
            t = (w >> (4 * i)) & 0x000F000F
            out += [t & 0xF, (t >> 16) & 0xF]
    return out


@pytest.mark.parametrize("operand,view", [("i8", _consumer_view_i8), ("f16", _consumer_view_f16)])
def test_pb_v1_consumer_order(operand, view):
    N, K = 32, 256
    w = _random_logical(N, K, 11)
    codes = O.nibbles(w, K)
    words = O.prepack_B(w, N, K, operand).view(np.uint32)
    KB = K // 128
    for nb in range(N // 16):
        for kb in range(KB):
            blk = words[(nb * KB + kb) * 256:(nb * KB + kb + 1) * 256].reshape(64, 4)
            for lane in range(64):
                r, kq = lane % 16, lane // 16
                got = view([int(x) for x in blk[lane]])
                k0 = kb * 128 + kq * 32
                assert got == codes[nb * 16 + r, k0:k0 + 32].tolist()


def test_f16_class_word_equals_printed_exllama_packing():
    with open(os.path.join(GOLDEN, "exllama_word.json")) as f:
        g = json.load(f)
    # the shift table printed next to the kernel: (j // 2) * 4 + (j % 2) * 16
    assert g["shifts"] == [(j // 2) * 4 + (j % 2) * 16 for j in range(8)]
    N, K = 16, 128
    for case in g["cases"]:
        vals = np.zeros((N, K), dtype=np.uint8)
        vals[0, :8] = case["vals"]
        w = (vals[:, 0::2] | (vals[:, 1::2] << 4)).astype(np.uint8)
        words = O.prepack_B(w, N, K, "f16").view(np.uint32)
        # (n=0, k=0..7) is lane 0, word 0 of block 0
        assert int(words[0]) == int(case["expected_word"], 16)


def test_prepack_is_type_agnostic():
    """Prepack only moves bits: INT4 and UINT4B8 weights with the same codes
    pack identically (the bias-8 view differs from the two's complement view
    only by flipping bit 3 of every code, which commutes with the shuffle)."""
    N, K = 32, 256
    w = _random_logical(N, K, 5)
    flipped = w ^ np.uint8(0x88)
    a = O.prepack_B(w, N, K, "i8").view(np.uint32)
    b = O.prepack_B(flipped, N, K, "i8").view(np.uint32)
    assert np.array_equal(a ^ np.uint32(0x88888888), b)
    assert np.array_equal(O.weight_values(w, K, "int4"), O.weight_values(flipped, K, "uint4b8"))


def test_public_prepack_entry():
    N, K = 16, 128
    w = _random_logical(N, K, 3)
    assert np.array_equal(oracle.prepack_B(w, N, K, "i8"), O.prepack_B(w, N, K, "i8"))


def test_exllama_unshuffle_matches_printed_packing():
    """The golden words were evaluated by hand from the printed packing
    expression; unshuffling each must give back its eight values in k order."""
    with open(os.path.join(GOLDEN, "exllama_word.json")) as f:
        g = json.load(f)
    N, K = 1, 8
    for case in g["cases"]:
        word = np.array([int(case["expected_word"], 16)], dtype=np.uint32)
        logical = O.exllama_to_logical(word, N, K)
        got = [int(logical[0, k // 2] >> (4 * (k % 2))) & 0xF for k in range(8)]
        assert got == case["vals"]


def test_exllama_import_of_f16_class_is_a_word_relocation():
    """The ExLlama order is the F16-class word order, so importing for fp16 /
    bf16 GEMMs moves whole words: PB-v1 word (block, lane, kw) is source word
    (n, k / 8) of its lane's k range, unchanged."""
    N, K = 32, 384
    rng = np.random.default_rng(17)
    src = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    words = O.prepack_B_from_exllama(src, N, K, "f16").view(np.uint32)
    KB = K // 128
    for n in range(N):
        for w in range(K // 8):
            k = 8 * w
            kb, kq, kw = k // 128, (k % 128) // 32, (k % 32) // 8
            lane = 16 * kq + n % 16
            assert words[((n // 16) * KB + kb) * 256 + lane * 4 + kw] == src[n, w]


def test_exllama_import_equals_prepack_of_the_unpacked_codes():
    """Brute force on a small weight: pack random codes with the page's
    shuffle, one value at a time, then import; the result must equal
    prepacking the codes' logical bytes (both operand classes)."""
    N, K = 16, 256
    rng = np.random.default_rng(23)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    src = np.zeros((N, K // 8), dtype=np.uint32)
    for n in range(N):
        for k in range(K):
            j = k % 8
            src[n, k // 8] |= np.uint32(int(codes[n, k]) << ((j // 2) * 4 + (j % 2) * 16))
    logical = np.zeros((N, K // 2), dtype=np.uint8)
    for n in range(N):
        for k in range(K):
            logical[n, k // 2] |= np.uint8(int(codes[n, k]) << (4 * (k % 2)))
    for operand in ("i8", "f16"):
        assert np.array_equal(O.prepack_B_from_exllama(src, N, K, operand), O.prepack_B(logical, N, K, operand))
