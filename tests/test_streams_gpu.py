"""The bench's three-stream schedule (independent steps of the path on separate streams,
joined by events) gives bitwise the same outputs as the one-stream order: no step's
arithmetic depends on which stream or at what time it runs."""
import pytest
import torch

import bench
from tests.gpu_run import config_inputs, log, upload
from workloads import make_inputs, make_shape

pytestmark = pytest.mark.gpu


def _outputs(w, nstreams, passes=2):
    dev = torch.device("cuda:0")
    t = upload(w)
    r = bench.Runner(w, t, dev, nstreams=nstreams)
    outs = []
    for _ in range(passes):
        r.step()
        torch.cuda.synchronize()
        outs.append({k: v.clone() for k, v in r.buf.items()})
    return outs


@pytest.mark.parametrize("which", ["config3", "small"])
def test_three_streams_bitwise_equal_one_stream(which):
    if which == "config3":
        w = config_inputs(3)
    else:
        w = make_inputs(make_shape(700, [90, 1, 333, 64], 8, 2, 128, dtype="bf16"), seed=700)
    log(f"streams: {which} P={w.shape.P} lens={list(w.shape.lens)}")
    one = _outputs(w, 1)
    three = _outputs(w, 3)
    for a in one + three[1:]:
        for k in three[0]:
            assert torch.equal(a[k], three[0][k]), k
    log(f"  {len(three[0])} outputs bitwise equal over 2 passes each")
