"""Pins of the oracle's key-bitmap encoding of kept-key sets (meta-cache)."""
import numpy as np
import pytest

from oracle import ref


def test_hand_example():
    # keys 0, 5, 31 -> word 0 bits 0, 5, 31; keys 32, 33 -> word 1 bits 0, 1; key 70 -> word 2 bit 6
    idx = np.array([[0, 5, 31, 32, 33, 70, -1, -1]], dtype=np.int32)
    bits = ref.idx_to_bits(idx, n=71, topk=6)
    assert bits.shape == (1, 3)
    assert bits[0].tolist() == [(1 << 0) | (1 << 5) | (1 << 31), 0b11, 1 << 6]
    assert ref.bits_to_idx(bits, n=71, topk=6, kpad=8).tolist() == idx.tolist()


@pytest.mark.parametrize("n,k", [(1, 1), (37, 5), (64, 64), (1000, 205), (1000, 1), (1000, 1000)])
def test_round_trip_and_popcount(n, k):
    r = np.random.default_rng(n + k)
    kpad = ((k + 31) // 32) * 32
    idx = np.full((3, kpad), -1, np.int32)
    for i in range(3):
        idx[i, :k] = np.sort(r.choice(n, k, replace=False))
    bits = ref.idx_to_bits(idx, n, k)
    assert bits.shape == (3, (n + 31) // 32)
    assert [sum(bin(int(w)).count("1") for w in row) for row in bits] == [k] * 3
    assert np.array_equal(ref.bits_to_idx(bits, n, k, kpad), idx)


def test_bits_past_n_and_extra_keys_are_dropped():
    bits = np.array([[0xffffffff, 0xffffffff]], dtype=np.uint32)  # 64 bits set, n = 40
    out = ref.bits_to_idx(bits, n=40, topk=10, kpad=32)
    assert out[0, :10].tolist() == list(range(10)) and (out[0, 10:] == -1).all()
    short = ref.bits_to_idx(np.array([[0b101, 0]], dtype=np.uint32), n=40, topk=10, kpad=32)
    assert short[0, :2].tolist() == [0, 2] and (short[0, 2:] == -1).all()
