"""The bench's measurement probes (bench_probes.hip, a library of their own) do what their
timings assume: the stream probe reads every chunk and writes the selected ones where stated;
the MFMA probe runs."""
import numpy as np
import pytest
import torch

import bench_probes as N
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w", [32, 17, 1])
def test_stream_probe_writes_the_selected_chunks(w):
    say("probe stream w=%d" % w)
    dev = torch.device("cuda:0")
    chunks = 1000 * 32 + 7  # a ragged last group of 32 chunks
    src = torch.arange(chunks * 4, dtype=torch.int32, device=dev)
    dst_chunks = -(-chunks // 32) * w
    dst = torch.full((dst_chunks * 4,), -1, dtype=torch.int32, device=dev)
    out = torch.empty(3 * 256, dtype=torch.int32, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    N.check(N.lib().probe_stream(src.data_ptr(), chunks * 16, dst.data_ptr(), w, 3, out.data_ptr(), sp), "probe")
    torch.cuda.synchronize()
    s = src.view(-1, 4).cpu().numpy()
    d = dst.view(-1, 4).cpu().numpy()
    i = np.arange(chunks)
    sel = (i % 32) < w
    j = (i // 32) * w + (i % 32)
    assert np.array_equal(d[j[sel]], s[sel])
    written = np.zeros(dst_chunks, dtype=bool)
    written[j[sel]] = True
    assert (d[~written] == -1).all()  # slots of the ragged last group past the source stay untouched


def test_mfma_probe_accumulates():
    say("probe mfma")
    dev = torch.device("cuda:0")
    wg = 2
    # every code 0x2 (1.0) in both operands, scales 1: each accumulator gains 64 per MFMA K step
    ops = torch.full((wg * 256 * 32,), 0x22222222, dtype=torch.int32, device=dev)
    out = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    N.check(N.lib().probe_mfma(ops.data_ptr(), 3, wg, out.data_ptr(), sp), "probe")
    torch.cuda.synchronize()
    # a lane holds 16 accumulators of each of its 16 blocks: 256 values of 3 * 64
    assert torch.all(out == 256 * 3 * 64.0)
