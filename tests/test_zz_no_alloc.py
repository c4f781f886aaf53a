"""mx_grouped_mm_wgrad_noalloc (the wgrad for callers that cannot allocate) against
mx_grouped_mm_wgrad with a caller workspace: the same kernels and split decision, so
the outputs must agree bit for bit. Two split calls in a row share the library's
fixed scratch (the second smaller than the first), then a call that does not split."""

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_amd as mx
from mxfp8_block_scaled_amd import synth

from gpu_util import dev_bf16, dev_i32, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def _operands(rng, m, n, k):
    dy = dev_bf16(synth.normal_bf16(rng, (m, n), 1e-2))
    x = dev_bf16(synth.normal_bf16(rng, (m, k), 1.0))
    _, _, dytq, dyts = mx.mx_quantize_dim0_dim1(dy)
    _, _, xtq, xts = mx.mx_quantize_dim0_dim1(x)
    return dytq, dyts, xtq, xts


@pytest.mark.parametrize("out_dtype", [mx.MX_OUT_F32, mx.MX_OUT_BF16])
def test_noalloc_matches_workspace_call(out_dtype):
    rng = np.random.default_rng(91 + out_dtype)
    cases = [
        # the 576-wide dense layer's wgrad over 16384 tokens: 5 splits, 47 MB of partials
        (16384, 576, 4096, None),
        # smaller, grouped (one group empty, one ending off a 256-token window): 2 splits
        (4096, 288, 512, [1056, 0, 3040]),
        # enough output tiles (2 x 16 x 16): no split, no scratch
        (1024, 4096, 4096, [512, 512]),
    ]
    for m, n, k, sizes in cases:
        offs = None if sizes is None else dev_i32(np.cumsum(sizes).astype(np.int32))
        G = 1 if sizes is None else len(sizes)
        need = mx.mx_grouped_mm_wgrad_workspace_bytes(G, m, n, k)
        say(f"[noalloc] m={m} n={n} k={k} groups={G} split workspace {need} bytes")
        assert (need > 0) == (n < 4096)
        assert need <= mx.MX_WGRAD_NOALLOC_SCRATCH_BYTES
        ops = _operands(rng, m, n, k)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda:0")
        ref = mx.mx_grouped_mm_wgrad(*ops, offs, m, n, k, groups=G, out_dtype=out_dtype, workspace=ws)
        dt = torch.float32 if out_dtype == mx.MX_OUT_F32 else torch.bfloat16
        out = torch.full((G, n, k), float("nan"), dtype=dt, device="cuda:0")
        got = mx.mx_grouped_mm_wgrad_noalloc(*ops, offs, m, n, k, groups=G, out_dtype=out_dtype, out=out)
        assert got is out
        bits = torch.int32 if out_dtype == mx.MX_OUT_F32 else torch.int16
        assert torch.equal(got.view(bits), ref.view(bits)), f"m={m} n={n} k={k}: not bit-identical"
        if sizes is not None:
            for g, s in enumerate(sizes):
                if s == 0:
                    assert not torch.any(got[g] != 0)
