"""Key bitmaps of the compact meta-cache on the GPU, through the C ABI: encode
equals the oracle bit for bit, decode equals the oracle (including bitmaps with
more or fewer than K keys and stray bits past n), and decode(encode(idx)) is
idx at every size, up to the 118,800-token shape."""
import numpy as np
import pytest
import torch

import sparse_attention_diffusion_amd as mcs
from oracle import ref

pytestmark = pytest.mark.gpu


def _lists(heads, n, k, seed, dev):
    """Random ascending K-subsets of [0, n) per (head, group), -1 padded."""
    g = -(-n // mcs.GROUP)
    kpad = mcs.kpad_for(k)
    gen = torch.Generator(device=dev).manual_seed(seed)
    out = torch.full((heads, g, kpad), -1, dtype=torch.int32, device=dev)
    rows = out.view(-1, kpad)
    step = max(1, (1 << 28) // max(n, 1))  # rows per chunk of random keys
    for r0 in range(0, rows.shape[0], step):
        r1 = min(rows.shape[0], r0 + step)
        pick = torch.rand((r1 - r0, n), generator=gen, device=dev).argsort(dim=1)[:, :k]
        rows[r0:r1, :k] = pick.sort(dim=1).values.to(torch.int32)
    return out


def _u32(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("heads,n,k", [(1, 1, 1), (2, 37, 5), (2, 64, 64), (3, 1000, 205), (2, 1000, 1),
                                       (2, 1000, 1000), (2, 4097, 819)])
def test_encode_decode_match_oracle(heads, n, k):
    dev = torch.device("cuda:0")
    print(f"keybits encode/decode heads={heads} n={n} k={k}", flush=True)
    idx = _lists(heads, n, k, seed=n * 7 + k, dev=dev)
    bits = mcs.mcs_idx_to_bits(idx, n, k)
    back = mcs.mcs_bits_to_idx(bits, n, k)
    torch.cuda.synchronize()
    want_bits = ref.idx_to_bits(idx.cpu().numpy(), n, k)
    assert np.array_equal(_u32(bits), want_bits)
    assert np.array_equal(back.cpu().numpy(), ref.bits_to_idx(want_bits, n, k, idx.shape[2]))
    assert torch.equal(back, idx)


@pytest.mark.parametrize("n,k,p", [(1000, 205, 0.1), (1000, 205, 0.4), (37, 5, 0.5), (4097, 64, 0.02)])
def test_decode_of_arbitrary_bitmaps_matches_oracle(n, k, p):
    """Bitmaps with more or fewer than K set bits and set bits at or past n."""
    dev = torch.device("cuda:0")
    print(f"keybits decode arbitrary n={n} k={k} p={p}", flush=True)
    g, w = -(-n // mcs.GROUP), mcs.bits_words(n)
    rng = np.random.default_rng(n + k)
    on = rng.random((2, g, w, 32)) < p
    words = (on.astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)
    bits = torch.from_numpy(words.view(np.int32)).to(dev)
    kpad = mcs.kpad_for(k) + 32
    got = mcs.mcs_bits_to_idx(bits, n, k, kpad=kpad)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref.bits_to_idx(words, n, k, kpad))


def test_round_trip_at_118800_tokens():
    """Two heads of the 118,800-token shape at density 0.15 (K = 17,820): the
    round trip over all 3,714 rows, and the oracle on sampled rows."""
    dev = torch.device("cuda:0")
    n, k, heads = 118800, 17820, 2
    print(f"keybits round trip heads={heads} n={n} k={k}", flush=True)
    idx = _lists(heads, n, k, seed=5, dev=dev)
    bits = mcs.mcs_idx_to_bits(idx, n, k)
    back = mcs.mcs_bits_to_idx(bits, n, k)
    torch.cuda.synchronize()
    assert torch.equal(back, idx)
    flat_idx, flat_bits = idx.view(-1, idx.shape[2]), bits.view(-1, bits.shape[2])
    for r in (0, 1, 1856, 1857, 3000, flat_idx.shape[0] - 1):
        want = ref.idx_to_bits(flat_idx[r:r + 1].cpu().numpy(), n, k)
        assert np.array_equal(_u32(flat_bits[r:r + 1]), want), r
