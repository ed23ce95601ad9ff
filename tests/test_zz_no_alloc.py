"""mcs_select_noalloc, the selection entry point without a workspace argument (its
intermediates live in the library's static device scratch), against mcs_select
on the same inputs: index lists must be identical, bit for bit, on consecutive
calls that shrink and grow the workload (the scratch keeps the previous call's
contents), with pass 1 in the kernel and with a supplied logsumexp."""
import numpy as np
import pytest
import torch

import sparse_attention_diffusion_amd as mcs
from sparse_attention_diffusion_amd import workloads as W
from tests.gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


def _case(heads, grid, d, dtype, seed):
    wl = W.Workload("t", grid, heads, d, dtype, 64, (0.2,), seed, 0.0, 0)
    q, k, _ = W.make_qkv(wl)
    n = q.shape[1]
    perm = np.stack([np.random.default_rng(seed + h).permutation(n) for h in range(heads)]).astype(np.int32)
    return to_dev(q, dtype), to_dev(k, dtype), torch.from_numpy(perm).to(dev())


@pytest.mark.parametrize("with_lse", [False, True])
def test_noalloc_select_matches_workspace_select(with_lse):
    # 3 heads x 2,040 tokens, then a smaller 2 x 770 fp32 case, then a larger one again
    cases = [((3, (6, 17, 20), 128, "bf16", 3), 0.15), ((2, (5, 11, 14), 64, "f32", 4), 0.3),
             ((4, (8, 19, 21), 128, "bf16", 5), 0.2)]
    for (heads, grid, d, dtype, seed), rho in cases:
        q, k, perm = _case(heads, grid, d, dtype, seed)
        n = q.shape[1]
        kk = max(1, int(round(rho * n)))
        lse = mcs.mcs_dense_attn(q, k, k, want_lse=True)[1] if with_lse else None
        want = mcs.mcs_select(q, k, perm, kk, lse=lse)
        got = mcs.mcs_select_noalloc(q, k, perm, kk, lse=lse)
        torch.cuda.synchronize()
        print(f"heads={heads} n={n} d={d} {dtype} K={kk} lse={'supplied' if with_lse else 'pass 1'}", flush=True)
        assert torch.equal(got, want), (heads, n, d, dtype, kk)
        assert (got[:, :, kk:] == -1).all()


def test_noalloc_rejects_a_workload_beyond_its_scratch():
    # one head of 50,000 tokens needs 782 mass rows of 50,000 fp32 (156 MB) > 128 MiB
    q = torch.zeros((1, 50000, 64), dtype=torch.bfloat16, device=dev())
    perm = torch.zeros((1, 50000), dtype=torch.int32, device=dev())
    with pytest.raises(mcs.McsError, match="scratch"):
        mcs.mcs_select_noalloc(q, q, perm, 100)
