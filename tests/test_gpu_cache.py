"""Meta-cache on the GPU: the host round trip is the identity, and a trajectory
with offload + prefetch (with list or compact bitmap entries, and with some
layers kept resident) produces bit-identical outputs to the all-resident one."""
import numpy as np
import pytest
import torch

import sparse_attention_diffusion_amd as mcs
from sparse_attention_diffusion_amd import trajectory
from sparse_attention_diffusion_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_copy_round_trip_is_bitwise():
    dev = torch.device("cuda:0")
    x = torch.randint(-2**31, 2**31 - 1, (3, 1000, 37), dtype=torch.int32, device=dev)
    host = torch.empty(x.shape, dtype=torch.int32, pin_memory=True)
    back = torch.empty_like(x)
    side = torch.cuda.Stream(device=dev)
    ev = torch.cuda.Event()
    side.wait_stream(torch.cuda.current_stream(dev))
    mcs.mcs_copy_async(host, x, mcs.MCS_COPY_D2H, stream=side)
    mcs.mcs_copy_async(back, host, mcs.MCS_COPY_H2D, stream=side)
    ev.record(side)
    torch.cuda.current_stream(dev).wait_event(ev)
    torch.cuda.synchronize()
    assert torch.equal(back, x)


@pytest.mark.parametrize("compact,resident,layers", [(False, 0, 3), (True, 0, 3), (True, 1, 4), (False, 2, 4)])
def test_offloaded_trajectory_matches_resident_bitwise(compact, resident, layers):
    print(f"trajectory offload compact={compact} resident layers={resident} of {layers}", flush=True)
    wl = W.Workload("traj_small", (4, 8, 20), 2, 128, "bf16", 64, (0.2,), 11, 0.02, 0, layers=layers, steps=12)
    keys = {(s, l): None for s in (2, 3, 4, 7, 11) for l in range(layers)}
    rec_a, rec_b = dict(keys), dict(keys)
    ra = trajectory.run(wl, layers=layers, steps=12, warmup=2, interval=3, density=0.2, offload=False,
                        record_outputs=rec_a)
    rb = trajectory.run(wl, layers=layers, steps=12, warmup=2, interval=3, density=0.2, offload=True,
                        device_slots=2, record_outputs=rec_b, compact=compact, resident_layers=resident)
    assert rb["resident_layers"] == resident
    assert rb["bytes_d2h"] > 0
    # entries come back from the host only when the offloaded layers outnumber the device slots
    assert (rb["bytes_h2d"] > 0) == (layers - resident > 2)
    for key in keys:
        assert torch.equal(rec_a[key], rec_b[key]), key
    print({k: ra[k] for k in ("attention_ms", "speedup_vs_dense", "anchor_overhead_density_points")})
