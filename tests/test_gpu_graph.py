"""HIP graph capture of library calls: a captured sequence (one-pass and 32x32
casts, the fused padded cast, grouped forward, dgrad, and a split-contraction
wgrad) replayed several times, with other eager work and synchronisations between
the replays; every replay must reproduce the eager results bit for bit.

The calls enqueue kernels only (no memset nodes, no host synchronisation, no
allocation by the library): the sequence is captured before it has ever run (no
warm-up call); the split-contraction wgrad's workspace is the caller's (here a
torch allocation from the graph's own memory pool). Between the replays a larger
split wgrad runs eagerly with a workspace of its own, which must not disturb them.
"""

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


def test_captured_sequence_replays():
    rng = np.random.default_rng(71)
    m, n, k, G = 4096, 576, 512, 4
    sizes = np.array([1024, 0, 1536, 1536])
    offs = dev_i32(synth.offs_from_sizes(sizes))
    raw_offs = dev_i32(np.cumsum([1000, 3, 1600, 1493]).astype(np.int32))  # unaligned, for the padded path
    x = dev_bf16(synth.normal_bf16(rng, (m, k), 1.0))
    w = dev_bf16(synth.normal_bf16(rng, (G * n, k), 0.02))
    dy = dev_bf16(synth.normal_bf16(rng, (m, n), 1e-2))
    wn = dev_bf16(synth.normal_bf16(rng, (n, k), 0.02))
    rows_pad = mx.mx_padded_rows(m, G)
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda:0")  # noqa: E731
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda:0")  # noqa: E731
    sb = mx.mx_scale_bytes
    b = {"xq": u8(m, k), "xs": u8(sb(m, k)), "xtq": u8(k, m), "xts": u8(sb(k, m)),
         "wq": u8(G * n, k), "ws": u8(sb(G * n, k)),
         "dyq": u8(m, n), "dys": u8(sb(m, n)), "dytq": u8(n, m), "dyts": u8(sb(n, m)),
         "pq": u8(rows_pad, k), "ps": u8(sb(rows_pad, k)), "ptq": u8(k, rows_pad), "pts": u8(sb(k, rows_pad)),
         "poffs": torch.empty(G, dtype=torch.int32, device="cuda:0"),
         "y": bf(m, n), "dx": bf(m, k), "dw": torch.empty((G, n, k), dtype=torch.float32, device="cuda:0"),
         "yp": bf(m, n)}

    def sequence():
        mx.mx_quantize_dim0_dim1(x, b["xq"], b["xs"], b["xtq"], b["xts"])
        mx.mx_quantize_dim0(w, b["wq"], b["ws"])
        mx.mx_quantize_dim0_dim1(dy, b["dyq"], b["dys"], b["dytq"], b["dyts"])
        b["nq"], b["nqt"], b["nsr"], b["nsc"] = mx.mx_quantize_weight_32x32(wn)
        mx.mx_grouped_mm_fwd(b["xq"], b["xs"], b["wq"], b["ws"], offs, m, n, k, out=b["y"])
        mx.mx_grouped_mm_dgrad(b["dyq"], b["dys"], b["nqt"], b["nsc"], None, m, n, k, out=b["dx"])
        # 576 x 512 outputs per group: 24 tiles, so each group's contraction is split two
        # ways (workspace + reduction)
        mx.mx_grouped_mm_wgrad(b["dytq"], b["dyts"], b["xtq"], b["xts"], offs, m, n, k, out=b["dw"],
                               out_dtype=mx.MX_OUT_F32)
        mx.mx_pad_quantize_dim0_dim1(x, raw_offs, rows_pad, b["pq"], b["ps"], b["ptq"], b["pts"], b["poffs"])
        mx.mx_grouped_mm_fwd_padded(b["pq"], b["ps"], b["wq"], b["ws"], b["poffs"], raw_offs, rows_pad, m, n, k,
                                    out=b["yp"])

    outs = ("xq", "xts", "dyq", "nqt", "nsc", "y", "dx", "dw", "pq", "pts", "poffs", "yp")
    g = torch.cuda.CUDAGraph()
    say("[graph] capture (no warm-up call)")
    with torch.cuda.graph(g):
        sequence()
    torch.cuda.synchronize()
    captured = {key: b[key] for key in outs}  # the 32x32 cast returns new tensors on every call
    say("[graph] eager reference")
    for key in outs:
        b[key].zero_()
    sequence()
    torch.cuda.synchronize()
    ref = {key: b[key].clone() for key in outs}
    b.update(captured)
    # a larger split wgrad between the replays: 576 x 1024 outputs over 16384 tokens
    big_m, big_k = 16384, 1024
    bx = dev_bf16(synth.normal_bf16(rng, (big_m, big_k), 1.0))
    bdy = dev_bf16(synth.normal_bf16(rng, (big_m, n), 1e-2))
    _, _, bxtq, bxts = mx.mx_quantize_dim0_dim1(bx)
    _, _, bdytq, bdyts = mx.mx_quantize_dim0_dim1(bdy)
    need = mx.mx_grouped_mm_wgrad_workspace_bytes(1, big_m, n, big_k)
    assert need > mx.mx_grouped_mm_wgrad_workspace_bytes(G, m, n, k) > 0
    big_ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    for r in range(3):
        for key in outs:
            b[key].zero_()
        mx.mx_grouped_mm_wgrad(bdytq, bdyts, bxtq, bxts, None, big_m, n, big_k, out_dtype=mx.MX_OUT_F32,
                               workspace=big_ws)
        torch.cuda.synchronize()
        say(f"[graph] replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for key in outs:
            assert torch.equal(b[key], ref[key]), f"replay {r}: {key} differs from the eager result"
