"""The allocation-free inference forward (gemm_fp4_bf16_fwd_qw_noalloc) against the entry point
it varies, gemm_fp4_bf16_fwd_qw with training = 0 and a caller workspace: two calls in a row,
the second with a smaller input (the library's scratch array keeps the first call's contents),
each bit-identical to the workspace form and within the GEMM bar of the oracle; the same for
two calls whose GEMMs split their contraction (partials in the scratch array as well).  Also:
sizes past the scratch array are rejected before anything runs."""
import numpy as np
import pytest
import torch

import oracle
import mxfp4_block_scaled_cast_amd as mx
from mxfp4_block_scaled_cast_amd import _native as native
from mxfp4_block_scaled_cast_amd import workloads as W
from gpu_util import say, to_device, bf16_to_f64, assert_gemm_close

pytestmark = pytest.mark.gpu


def stream():
    return torch.cuda.current_stream().cuda_stream


def run_pair(M, N, K, seed):
    a = W.ragged_values((M, K), seed)
    w = W.ragged_values((N, K), seed + 1)
    L = native.lib()
    Wt = mx.cast_dual(to_device(w))
    ad = to_device(a)
    ref_out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    nbytes = L.gemm_fp4_bf16_workspace_bytes_qw(M, N, K, 0)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device="cuda:0")
    say("gemm_fp4_bf16_fwd_qw (workspace) M=%d N=%d K=%d" % (M, N, K))
    native.check(L.gemm_fp4_bf16_fwd_qw(ad.data_ptr(), Wt.row.q.data_ptr(), Wt.row.s.data_ptr(), M, N, K,
                                        ref_out.data_ptr(), ws.data_ptr(), nbytes, 0, stream()), "fwd_qw")
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    say("gemm_fp4_bf16_fwd_qw_noalloc M=%d N=%d K=%d" % (M, N, K))
    native.check(L.gemm_fp4_bf16_fwd_qw_noalloc(ad.data_ptr(), Wt.row.q.data_ptr(), Wt.row.s.data_ptr(), M, N, K,
                                                out.data_ptr(), stream()), "fwd_qw_noalloc")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    qa, sa = oracle.cast_rows(a)
    qw, sw = oracle.cast_rows(w)
    ref, absref = oracle.gemm(qa, sa, qw, sw)
    assert_gemm_close(bf16_to_f64(out), ref, absref, "noalloc %dx%dx%d" % (M, N, K))


def test_two_calls_second_smaller():
    # first: persistent tiled GEMM (2048 x 4096 = 128 tiles), A's row copy 1.1 MB; second: a
    # ragged skinny shape whose row copy is a fraction of the first one left in the array
    run_pair(2048, 4096, 512, 501)
    run_pair(17, 160, 288, 503)


def test_split_contractions_through_the_scratch():
    # the split partials live in the scratch array too: first a 128 x 8192 output over 8192 on the
    # panel kernel (4 splits, 16 MiB of partials after A's row copy), then a smaller 17 x 1024 output
    # over 20480 on the skinny kernel (its partials where the first call's were)
    assert mx.gemm_workspace_bytes(128, 8192, 8192) > 0 and mx.gemm_workspace_bytes(17, 1024, 20480) > 0
    run_pair(128, 8192, 8192, 507)
    run_pair(17, 1024, 20480, 509)


def test_sizes_past_the_scratch_are_rejected():
    L = native.lib()
    M, K = 16384, 8192  # A's row copy: 71 MB > 64 MiB
    assert L.gemm_fp4_bf16_workspace_bytes_qw(M, 64, K, 0) > native.NOALLOC_SCRATCH_BYTES
    assert L.gemm_fp4_bf16_fwd_qw_noalloc(1 << 20, 1 << 20, 1 << 20, M, 64, K, 1 << 20, None) == -5
    assert L.gemm_fp4_bf16_fwd_qw_noalloc(1 << 20, 1 << 20, 1 << 20, 64, 64, 48, 1 << 20, None) == -1
    assert L.gemm_fp4_bf16_fwd_qw_noalloc(None, 1 << 20, 1 << 20, 0, 64, 64, None, None) == 0
