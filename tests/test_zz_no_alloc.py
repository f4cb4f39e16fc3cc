"""vsa_select_noalloc, the selector without a workspace argument (for callers
that cannot allocate device memory), against vsa_select: two calls in a row
through the C ABI, the second on a smaller input, each bit-equal to
vsa_select's ids on the same input (same kernels, same arithmetic; only the
scratch and the grouping of (batch, head) pairs into launches differ)."""
import numpy as np
import pytest
import torch

import video_dit_block_amd as vsa
from video_dit_block_amd import _lib

pytestmark = pytest.mark.gpu


def _inputs(B, Nc, NH, D, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((B, Nc * 64, NH, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Nc * 64, NH, D), generator=g, device="cuda").to(torch.bfloat16)
    vbs = torch.randint(1, 65, (Nc,), generator=g, device="cuda", dtype=torch.int32)
    return q, k, vbs


def _check(q, k, vbs, topk, label):
    B, S, NH, D = q.shape
    Nc = S // 64
    print(f"[{label}] B={B} Nc={Nc} NH={NH} D={D} topk={topk}", flush=True)
    ref = vsa.select(q, k, vbs, topk)
    out = torch.full((B, NH, Nc, topk), -7, dtype=torch.int32, device="cuda")
    st = _lib.load().vsa_select_noalloc(q.data_ptr(), k.data_ptr(), vbs.data_ptr(), B, Nc, NH, D,
                                        topk, out.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "vsa_select_noalloc")
    torch.cuda.synchronize()
    a, r = out.cpu().numpy(), ref.cpu().numpy()
    print(f"[{label}] differing ids: {int((a != r).sum())} of {a.size}", flush=True)
    assert np.array_equal(a, r), label


def test_noalloc_select_two_calls_bit_equal():
    # call 1: the Wan shape (624 cubes, 40 heads of 128: two chunks of heads),
    # two batches; call 2: smaller, D = 64, one chunk
    q, k, vbs = _inputs(2, 624, 40, 128, seed=3)
    _check(q, k, vbs, 78, "noalloc wan-shaped")
    del q, k
    q, k, vbs = _inputs(1, 24, 3, 64, seed=4)
    _check(q, k, vbs, 5, "noalloc small")
