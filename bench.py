"""Benchmark: one MXFP8 MoE training step (casts + grouped GEMM forward, dgrad,
wgrad) on one MI355X, printed as one JSON line.

Workload (the pages' grouped-GEMM benchmark shape, pytorch/ao PR 4705 "Wire MoE
and MXFP8Linear training paths to CuTeDSL by default", grouped benchmark command:
K=N=4096, G=8, M=16384): tokens X [16384, 4096] ~ N(0,1), expert weights
W [8, 4096, 4096] ~ N(0,0.02), grad_out dY [16384, 4096] ~ N(0,1e-2), multinomial
group sizes in multiples of 32; plus the unaligned dense layer of the 576-wide
gradient (torchtitan PR 5334, body): W' [576, 4096] with 32x32 weight scales and
dY' [16384, 576]. Synthetic, seeded data; inputs resident in HBM before timing.

One step runs, in order:
  dim0 X, dim0 W (3D as rows), grouped fwd           -> Y  [16384, 4096] bf16
  dim0 dY, dim1 W (3D batched), grouped dgrad         -> dX [16384, 4096] bf16
  dim1 dY, dim1 X, grouped wgrad                      -> dW [8, 4096, 4096] bf16
  32x32 W', dense fwd (reuses dim0 X)                 -> Y' [16384, 576] bf16
  dim0 dY', dense dgrad over the 576-wide contraction -> dX' [16384, 4096] bf16
  dim1 dY', dense wgrad (reuses dim1 X)               -> dW' [576, 4096] bf16
`value` = all GEMM flops of the step / step time (casts included).

--unaligned-groups: the same tokens with per-row (not 32-aligned) group sizes;
the step pads X and dY to 32-row group boundaries inside the casts (ao fork PR 10,
"Known follow-ups": padded token groups), runs the grouped passes on the padded
rows and offsets, fwd and dgrad writing Y and dX unpadded; flops count real rows
only.

--backward ARM: the MoE grouped step (no dense layer) with the backward override
arm ARM (ao fork PR 10, "Design notes"): "quantized" (the MXFP8 backward),
"high_precision" (transposes of the saved bf16 W, X, dY and bf16 grouped GEMMs) or
"dequantized" (the forward's codes of W and X dequantized transposed, dY
transposed, bf16 grouped GEMMs); bf16 GEMMs are priced against the bf16 peak.

--workload deepseek_share: one GPU's expert share of a DeepSeek-V3-like MoE layer
(32 experts, hidden 7168, expert FFN 2048, 4096 tokens x top-8 = 32768 routed
rows, Zipf(1.2) group sizes with 3 experts empty): one-pass casts of X, W1, H,
W2, dY2, dY1 and the grouped fwd, dgrad and wgrad of the gate/up projection
(W1 [32, 4096, 7168]) and the down projection (W2 [32, 7168, 2048]). No CPU
baseline in this mode; `traffic` is the committed counter figure of its gate/up wgrad.

--precise: the default step with its six GEMMs computed from the same codes on the
bf16 MFMA (both operands dequantized to bf16 inside each op, then the bf16 grouped
GEMM): the route whose fp32 outputs meet the IEEE-fp32 figure, priced against the
bf16 peak.

--cycle-stamps: loads the instrumented build (libmxfp8_stamps.so) and prints each GEMM
launch's per-block cycle breakdown instead of a timing line.

--workload linear_4096: the dense MXFP8Linear step of the linear benchmark command on
"Wire MoE and MXFP8Linear training paths to CuTeDSL by default" (M=N=4096, K=2048,
CUDA-graph replay): one-pass casts of X [4096, 2048] and dY [4096, 4096], the 32x32
cast of W [4096, 2048] (both orientations), then fwd Y = X W^T, dgrad dX = dY W (W^T
from the 32x32 cast) and wgrad dW = dY^T X; 206.2 GFLOP per step. The step is captured
into a HIP graph of `steps` steps (100 by default) and replayed once as the timed
region; the dominant kernel is timed by events around its eager launches right after.
The 256^3 small linear (dim0 casts of
A and B with their planted zero and outlier blocks, fwd with fp32 output) is timed the
same way and reported as a latency beside it. The CPU baseline is the oracle on the
whole step.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 grouped GEMM TFLOP/s (fwd+bwd) and cast GB/s vs roofline, 1 GPU"
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 / MXFP8 MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAKS = {"gemm": PEAK_FP8_TFLOPS, "gemm16": PEAK_BF16_TFLOPS}
PEAK_HBM_GBPS = 8000.0
CAST_BYTES_PER_ELEM = 2 + 1 + 1 / 32  # read bf16, write e4m3 + one scale byte per 32
W32_BYTES_PER_ELEM = 2 + 1 + 1 + 2 / 32  # both orientations, row and column scales
BOTH_BYTES_PER_ELEM = 2 + 1 + 1 + 2 / 32  # one-pass dim0 + dim1: read once, both codes and scales
M, K, N, G, NARROW = 16384, 4096, 4096, 8, 576


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # 100 untimed steps (~0.13 s): after 5 the timed steps still ran ~7% slower (1.366-1.371 against
    # 1.274-1.283 ms, same device), the device still raising its clocks
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate-casts", action="store_true",
                    help="cast each tensor with separate dim0 and dim1 kernels instead of the one-pass cast")
    ap.add_argument("--only", default=None,
                    help="run only the ops of the step whose name contains this text (for counter runs)")
    ap.add_argument("--unaligned-groups", action="store_true",
                    help="group sizes drawn per row (not multiples of 32): the step pads X and dY to 32-row "
                         "group boundaries, runs the grouped passes on the padded offsets and unpads Y and dX")
    ap.add_argument("--backward", default=None, choices=["quantized", "high_precision", "dequantized"],
                    help="time the MoE grouped step (forward + the named backward override arm) instead")
    ap.add_argument("--workload", default="moe_g8", choices=["moe_g8", "deepseek_share", "linear_4096"],
                    help="deepseek_share: one GPU's share of a DeepSeek-V3-like MoE layer (32 experts, hidden "
                         "7168, FFN 2048, 32768 routed rows, Zipf group sizes, 3 experts empty), fwd+bwd of "
                         "both expert projections, instead of the default MoE step; linear_4096: the dense "
                         "MXFP8Linear fwd+bwd at M=N=4096, K=2048 (32x32 weight scales) replayed as a HIP graph, "
                         "with the 256^3 small linear's latency beside it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device-to-device copy instead (reference for HBM byte counters)")
    ap.add_argument("--precise", action="store_true",
                    help="the default step with its six GEMMs computed from the same codes on the bf16 MFMA "
                         "(mxfp8_block_scaled_amd.precise: dequantize both operands, bf16 grouped GEMM), the "
                         "path that meets the IEEE-fp32 figure; priced against the bf16 peak")
    ap.add_argument("--cycle-stamps", action="store_true",
                    help="load the instrumented library (libmxfp8_stamps.so), run the step, then each GEMM of "
                         "the step once more alone and print its per-block cycle breakdown as one JSON line")
    return ap.parse_args()


HASHED_SOURCES = ("gemm.hip", "cast.hip", "common.h", "group_table.h")


def src_hash(csrc=None):
    """Hash of the GEMM and cast kernel sources with comments and whitespace removed,
    and without the blocks that only the instrumented build (MX_CYCLE_STAMPS)
    compiles: the counters in profiles/traffic.json hold while it matches."""
    csrc = csrc or os.path.join(ROOT, "mxfp8_block_scaled_amd", "csrc")
    h = hashlib.sha256()
    for f in HASHED_SOURCES:
        with open(os.path.join(csrc, f)) as fh:
            text = fh.read()
        text = re.sub(r"#ifdef MX_CYCLE_STAMPS\n.*?#endif\n", "", text, flags=re.S)
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, units_per_launch):
    """HBM bytes per launch from the committed counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != src_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def wgrad_workspace(mx, dev, groups, m, n, k, bf16=False):
    """The caller-owned split-contraction workspace of one wgrad call (None if it does
    not split)."""
    import torch

    need = mx.mx_grouped_mm_wgrad_workspace_bytes(groups, m, n, k, bf16)
    return torch.empty(need, dtype=torch.uint8, device=dev) if need else None


def deepseek_share_ops(mx, synth, to_dev, dev):
    """The expert share's training step: one-pass casts of X, W1, H, W2, dY2, dY1 and the
    grouped fwd, dgrad and wgrad of the gate/up (X -> 4096) and down (H -> 7168)
    projections; 8.659 TFLOP of GEMMs per step."""
    import torch

    d = synth.deepseek_share(0)
    offs_np = d["offs"]
    t = {k: to_dev(v) for k, v in d.items() if k != "offs"}
    del d
    offs = torch.from_numpy(offs_np).to(dev)
    E, N1, H_ = t["w1"].shape  # 32, 4096, 7168
    _, _, F = t["w2"].shape     # 2048
    R = t["x"].shape[0]         # 32768 routed rows
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)  # noqa: E731
    sb = mx.mx_scale_bytes
    q = {}
    for name, (rows, cols, batch) in {"x": (R, H_, 1), "w1": (N1, H_, E), "h": (R, F, 1), "w2": (H_, F, E),
                                      "dy2": (R, H_, 1), "dy1": (R, N1, 1)}.items():
        q[name] = (u8(batch * rows, cols), u8(sb(batch * rows, cols)),
                   u8(cols, rows) if batch == 1 else u8(batch, cols, rows), u8(sb(batch * cols, rows)))
    y1, y2, dh, dx = bf(R, N1), bf(R, H_), bf(R, F), bf(R, H_)
    dw1, dw2 = bf(E, N1, H_), bf(E, H_, F)
    both = lambda n_elem: n_elem * BOTH_BYTES_PER_ELEM  # noqa: E731
    ws_down = wgrad_workspace(mx, dev, E, R, H_, F)
    ws_gate = wgrad_workspace(mx, dev, E, R, N1, H_)

    def cast(name):
        # inputs' and weights' transposed codes are read late (wgrad, dgrad): streamed;
        # the gradients' are read by the wgrad right after their dgrad: cached
        st = name in ("x", "w1", "h", "w2")
        return ("cast_dim0+dim1 " + name, "cast", both(t[name].numel()),
                lambda: mx.mx_quantize_dim0_dim1(t[name], *q[name], stream_t=st))

    ops = [
        cast("x"), cast("w1"),
        ("gemm_fwd gate/up", "gemm", 2 * R * N1 * H_,
         lambda: mx.mx_grouped_mm_fwd(q["x"][0], q["x"][1], q["w1"][0], q["w1"][1], offs, R, N1, H_, out=y1)),
        cast("h"), cast("w2"),
        ("gemm_fwd down", "gemm", 2 * R * H_ * F,
         lambda: mx.mx_grouped_mm_fwd(q["h"][0], q["h"][1], q["w2"][0], q["w2"][1], offs, R, H_, F, out=y2)),
        cast("dy2"),
        ("gemm_dgrad down", "gemm", 2 * R * H_ * F,
         lambda: mx.mx_grouped_mm_dgrad(q["dy2"][0], q["dy2"][1], q["w2"][2], q["w2"][3], offs, R, H_, F, out=dh)),
        ("gemm_wgrad down", "gemm", 2 * R * H_ * F,
         lambda: mx.mx_grouped_mm_wgrad(q["dy2"][2], q["dy2"][3], q["h"][2], q["h"][3], offs, R, H_, F, out=dw2,
                                        out_dtype=mx.MX_OUT_BF16, workspace=ws_down)),
        cast("dy1"),
        ("gemm_dgrad gate/up", "gemm", 2 * R * N1 * H_,
         lambda: mx.mx_grouped_mm_dgrad(q["dy1"][0], q["dy1"][1], q["w1"][2], q["w1"][3], offs, R, N1, H_, out=dx)),
        ("gemm_wgrad gate/up", "gemm", 2 * R * N1 * H_,
         lambda: mx.mx_grouped_mm_wgrad(q["dy1"][2], q["dy1"][3], q["x"][2], q["x"][3], offs, R, N1, H_, out=dw1,
                                        out_dtype=mx.MX_OUT_BF16, workspace=ws_gate)),
    ]
    config = {"workload": "deepseek_share fwd+dgrad+wgrad: 32 experts, hidden 7168, FFN 2048 (gate/up N=4096, "
                          "down N=7168 over K=2048), 32768 routed rows, Zipf(1.2) group sizes with 3 empty experts; "
                          "one-pass casts of X, W1, H, W2, dY2, dY1",
              "M": R, "K": H_, "N": N1, "G": E, "narrow": None, "offs": offs_np.tolist(), "rows_padded": None,
              "parallelism": "none (1 GPU)"}
    return ops, config


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "there is no multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mxfp8_block_scaled_amd as mx
    from mxfp8_block_scaled_amd import synth

    if args.cycle_stamps:
        # the instrumented build of the same sources; loaded before any library call
        from mxfp8_block_scaled_amd import _lib, build as _build

        assert os.path.exists(_build.STAMPS_LIB), "build it: python -m mxfp8_block_scaled_amd.build --stamps"
        _lib.LIB_PATH = _build.STAMPS_LIB

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": 1 << 30, "copies": args.warmup + args.steps}))
        return

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    if args.workload == "linear_4096":
        assert not (args.unaligned_groups or args.backward or args.separate_casts or args.only or args.cycle_stamps
                    or args.precise), \
            "--workload linear_4096 runs its own step"
        return linear_4096_main(args, mx, synth, to_dev, dev)

    d = synth.moe_g8(0, with_backward=True)
    offs_np = d["offs"]
    X, W, dY = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["dy"])
    Wn, dYn = to_dev(d["w_narrow"]), to_dev(d["dy_narrow"])
    del d
    unaligned = args.unaligned_groups
    if unaligned:
        # per-row multinomial group sizes; the grouped passes see the padded rows
        offs_np = np.cumsum(np.random.default_rng(1).multinomial(M, np.full(G, 1.0 / G))).astype(np.int32)
    offs = torch.from_numpy(offs_np).to(dev)
    Mg = mx.mx_padded_rows(M, G) if unaligned else M
    offs_pad = torch.empty(G, dtype=torch.int32, device=dev)
    goffs = offs_pad if unaligned else offs

    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
    sb = mx.mx_scale_bytes
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)  # noqa: E731
    buf = {
        "xq": u8(Mg, K), "xs": u8(sb(Mg, K)),
        "wq": u8(G * N, K), "ws": u8(sb(G * N, K)),
        "dyq": u8(Mg, N), "dys": u8(sb(Mg, N)),
        "wtq": u8(G, K, N), "wts": u8(sb(G * K, N)),
        "dytq": u8(N, Mg), "dyts": u8(sb(N, Mg)),
        "xtq": u8(K, Mg), "xts": u8(sb(K, Mg)),
        "y": bf(Mg, N), "dx": bf(Mg, K), "dw": bf(G, N, K),
        "dynq": u8(M, NARROW), "dyns": u8(sb(M, NARROW)),
        "dyntq": u8(NARROW, M), "dynts": u8(sb(NARROW, M)),
        "yn": bf(M, NARROW), "dxn": bf(M, K), "dwn": bf(1, NARROW, K),
    }
    Wflat = W.view(G * N, K)
    # split-contraction workspaces, allocated once outside the timed region
    ws = {"g": wgrad_workspace(mx, dev, G, Mg, N, K), "n": wgrad_workspace(mx, dev, 1, M, NARROW, K),
          "b": wgrad_workspace(mx, dev, G, M, N, K, bf16=True)}

    # (name, kind, work units, fn) ; kind "gemm" (MXFP8) / "gemm16" (bf16): units = flops,
    # "cast" / "pad": units = bytes
    cast0 = lambda n_elem: n_elem * CAST_BYTES_PER_ELEM  # noqa: E731
    both = lambda n_elem: n_elem * BOTH_BYTES_PER_ELEM  # noqa: E731
    w32 = {}

    def cast_w32():
        w32["q"], w32["qt"], w32["sr"], w32["sc"] = mx.mx_quantize_weight_32x32(Wn)

    # flops count the real token rows (padding rows are overhead, not work)
    g_fwd = ("gemm_fwd grouped", "gemm", 2 * M * N * K,
             lambda: mx.mx_grouped_mm_fwd(buf["xq"], buf["xs"], buf["wq"], buf["ws"], goffs, Mg, N, K,
                                          out=buf["y"]))
    g_dgrad = ("gemm_dgrad grouped", "gemm", 2 * M * N * K,
               lambda: mx.mx_grouped_mm_dgrad(buf["dyq"], buf["dys"], buf["wtq"], buf["wts"], goffs, Mg, N, K,
                                              out=buf["dx"]))
    g_wgrad = ("gemm_wgrad grouped", "gemm", 2 * M * N * K,
               lambda: mx.mx_grouped_mm_wgrad(buf["dytq"], buf["dyts"], buf["xtq"], buf["xts"], goffs, Mg, N, K,
                                              out=buf["dw"], out_dtype=mx.MX_OUT_BF16, workspace=ws["g"]))
    n_w32 = ("cast_w32 W'", "cast", NARROW * K * W32_BYTES_PER_ELEM, cast_w32)
    n_fwd = ("gemm_fwd dense576", "gemm", 2 * M * NARROW * K,
             lambda: mx.mx_grouped_mm_fwd(buf["xq"], buf["xs"], w32["q"], w32["sr"], None, M, NARROW, K,
                                          out=buf["yn"]))
    n_dgrad = ("gemm_dgrad dense576", "gemm", 2 * M * NARROW * K,
               lambda: mx.mx_grouped_mm_dgrad(buf["dynq"], buf["dyns"], w32["qt"], w32["sc"], None, M, NARROW, K,
                                              out=buf["dxn"]))
    n_wgrad = ("gemm_wgrad dense576", "gemm", 2 * M * NARROW * K,
               lambda: mx.mx_grouped_mm_wgrad(buf["dyntq"], buf["dynts"], buf["xtq"], buf["xts"], None, M, NARROW,
                                              K, out=buf["dwn"], out_dtype=mx.MX_OUT_BF16, workspace=ws["n"]))
    if args.precise:
        assert not (args.backward or unaligned or args.separate_casts or args.workload != "moe_g8"), \
            "--precise replaces the default MoE step's GEMMs only"
        from mxfp8_block_scaled_amd import precise

        # the same calls and operands; each op now also dequantizes its two operands
        g_fwd = ("precise fwd grouped", "gemm16", g_fwd[2],
                 lambda: precise.grouped_mm_fwd(buf["xq"], buf["xs"], buf["wq"], buf["ws"], goffs, Mg, N, K,
                                                out=buf["y"]))
        g_dgrad = ("precise dgrad grouped", "gemm16", g_dgrad[2],
                   lambda: precise.grouped_mm_dgrad(buf["dyq"], buf["dys"], buf["wtq"], buf["wts"], goffs, Mg, N, K,
                                                    out=buf["dx"]))
        g_wgrad = ("precise wgrad grouped", "gemm16", g_wgrad[2],
                   lambda: precise.grouped_mm_wgrad(buf["dytq"], buf["dyts"], buf["xtq"], buf["xts"], goffs, Mg, N,
                                                    K, out=buf["dw"], out_dtype=mx.MX_OUT_BF16))
        n_fwd = ("precise fwd dense576", "gemm16", n_fwd[2],
                 lambda: precise.grouped_mm_fwd(buf["xq"], buf["xs"], w32["q"], w32["sr"], None, M, NARROW, K,
                                                out=buf["yn"]))
        n_dgrad = ("precise dgrad dense576", "gemm16", n_dgrad[2],
                   lambda: precise.grouped_mm_dgrad(buf["dynq"], buf["dyns"], w32["qt"], w32["sc"], None, M, NARROW,
                                                    K, out=buf["dxn"]))
        n_wgrad = ("precise wgrad dense576", "gemm16", n_wgrad[2],
                   lambda: precise.grouped_mm_wgrad(buf["dyntq"], buf["dynts"], buf["xtq"], buf["xts"], None, M,
                                                    NARROW, K, out=buf["dwn"], out_dtype=mx.MX_OUT_BF16))
    if args.backward in ("high_precision", "dequantized"):
        # forward as MXFP8 (dim0 casts), backward from bf16 operands: transposes or
        # transposed dequantization (2 B written per element; 2 B read for bf16, 1 + 1/32
        # for codes) and bf16 grouped GEMMs
        wt16, xt16, dyt16 = bf(G, K, N), bf(K, M), bf(N, M)
        tb = lambda n_elem: 4 * n_elem  # noqa: E731
        db = lambda n_elem: n_elem * (2 + 1 + 1 / 32)  # noqa: E731
        if args.backward == "high_precision":
            w_src = ("transpose W", "cast", tb(G * N * K), lambda: mx.mx_transpose_bf16(W, wt16))
            x_src = ("transpose X", "cast", tb(M * K), lambda: mx.mx_transpose_bf16(X, xt16))
        else:
            w_src = ("dequant^T W", "cast", db(G * N * K),
                     lambda: mx.mx_dequantize(buf["wq"].view(G, N, K), buf["ws"], transpose=True, out=wt16))
            x_src = ("dequant^T X", "cast", db(M * K),
                     lambda: mx.mx_dequantize(buf["xq"], buf["xs"], transpose=True, out=xt16))
        ops = [
            ("cast_dim0 X", "cast", cast0(M * K), lambda: mx.mx_quantize_dim0(X, buf["xq"], buf["xs"])),
            ("cast_dim0 W", "cast", cast0(G * N * K), lambda: mx.mx_quantize_dim0(Wflat, buf["wq"], buf["ws"])),
            g_fwd,
            w_src,
            ("bf16 dgrad grouped", "gemm16", 2 * M * N * K,
             lambda: mx.mx_grouped_mm_bf16_dgrad(dY, wt16, offs, M, N, K, out=buf["dx"])),
            ("transpose dY", "cast", tb(M * N), lambda: mx.mx_transpose_bf16(dY, dyt16)),
            x_src,
            ("bf16 wgrad grouped", "gemm16", 2 * M * N * K,
             lambda: mx.mx_grouped_mm_bf16_wgrad(dyt16, xt16, offs, M, N, K, out=buf["dw"],
                                                 out_dtype=mx.MX_OUT_BF16, workspace=ws["b"])),
        ]
    elif args.backward == "quantized":
        ops = [
            ("cast_dim0+dim1 X", "cast", both(M * K),
             lambda: mx.mx_quantize_dim0_dim1(X, buf["xq"], buf["xs"], buf["xtq"], buf["xts"], stream_t=True)),
            ("cast_dim0+dim1 W", "cast", both(G * N * K),
             lambda: mx.mx_quantize_dim0_dim1(W, buf["wq"], buf["ws"], buf["wtq"], buf["wts"], stream_t=True)),
            g_fwd,
            ("cast_dim0+dim1 dY", "cast", both(M * N),
             lambda: mx.mx_quantize_dim0_dim1(dY, buf["dyq"], buf["dys"], buf["dytq"], buf["dyts"])),
            g_dgrad, g_wgrad,
        ]
    elif unaligned:
        # the MoE grouped part only (the dense layer has no groups). The padding is fused:
        # the casts read the real rows once and write the codes of every padded row
        # (bytes: 2 per real element read, 2 + 2/32 per padded element written); fwd and
        # dgrad write their outputs unpadded; wgrad contracts over the padded rows.
        padded_both = lambda n_real, n_pad: 2 * n_real + n_pad * (2 + 2 / 32)  # noqa: E731
        y_u, dx_u = bf(M, N), bf(M, K)
        ops = [
            # X's and W's transposed codes streamed past the caches, as in the aligned step
            ("cast_dim0+dim1 X (padded)", "cast", padded_both(M * K, Mg * K),
             lambda: mx.mx_pad_quantize_dim0_dim1(X, offs, Mg, buf["xq"], buf["xs"], buf["xtq"], buf["xts"],
                                                  offs_pad, stream_t=True)),
            ("cast_dim0+dim1 W", "cast", both(G * N * K),
             lambda: mx.mx_quantize_dim0_dim1(W, buf["wq"], buf["ws"], buf["wtq"], buf["wts"], stream_t=True)),
            ("gemm_fwd grouped", "gemm", 2 * M * N * K,
             lambda: mx.mx_grouped_mm_fwd_padded(buf["xq"], buf["xs"], buf["wq"], buf["ws"], offs_pad, offs, Mg, M,
                                                 N, K, out=y_u)),
            ("cast_dim0+dim1 dY (padded)", "cast", padded_both(M * N, Mg * N),
             lambda: mx.mx_pad_quantize_dim0_dim1(dY, offs, Mg, buf["dyq"], buf["dys"], buf["dytq"], buf["dyts"],
                                                  offs_pad)),
            ("gemm_dgrad grouped", "gemm", 2 * M * N * K,
             lambda: mx.mx_grouped_mm_dgrad_padded(buf["dyq"], buf["dys"], buf["wtq"], buf["wts"], offs_pad, offs,
                                                   Mg, M, N, K, out=dx_u)),
            g_wgrad,
        ]
    elif args.separate_casts:
        ops = [
            ("cast_dim0 X", "cast", cast0(M * K), lambda: mx.mx_quantize_dim0(X, buf["xq"], buf["xs"])),
            ("cast_dim0 W", "cast", cast0(G * N * K), lambda: mx.mx_quantize_dim0(Wflat, buf["wq"], buf["ws"])),
            g_fwd,
            ("cast_dim0 dY", "cast", cast0(M * N), lambda: mx.mx_quantize_dim0(dY, buf["dyq"], buf["dys"])),
            ("cast_dim1 W", "cast", cast0(G * N * K), lambda: mx.mx_quantize_dim1(W, buf["wtq"], buf["wts"])),
            g_dgrad,
            ("cast_dim1 dY", "cast", cast0(M * N), lambda: mx.mx_quantize_dim1(dY, buf["dytq"], buf["dyts"])),
            ("cast_dim1 X", "cast", cast0(M * K), lambda: mx.mx_quantize_dim1(X, buf["xtq"], buf["xts"])),
            g_wgrad,
            n_w32, n_fwd,
            ("cast_dim0 dY'", "cast", cast0(M * NARROW), lambda: mx.mx_quantize_dim0(dYn, buf["dynq"], buf["dyns"])),
            n_dgrad,
            ("cast_dim1 dY'", "cast", cast0(M * NARROW),
             lambda: mx.mx_quantize_dim1(dYn, buf["dyntq"], buf["dynts"])),
            n_wgrad,
        ]
    else:
        # every tensor here is needed in both orientations: one-pass casts. X's and W's
        # transposed codes are read only by wgrad and dgrad, after the forward and the dY
        # cast: they are streamed past the caches (MX_FORM_STREAM_T), which then still
        # hold X's and W's row-wise codes when the forward reads them; dY's transposed
        # codes are read by the wgrad right after dgrad and stay cached
        ops = [
            ("cast_dim0+dim1 X", "cast", both(M * K),
             lambda: mx.mx_quantize_dim0_dim1(X, buf["xq"], buf["xs"], buf["xtq"], buf["xts"], stream_t=True)),
            ("cast_dim0+dim1 W", "cast", both(G * N * K),
             lambda: mx.mx_quantize_dim0_dim1(W, buf["wq"], buf["ws"], buf["wtq"], buf["wts"], stream_t=True)),
            g_fwd,
            ("cast_dim0+dim1 dY", "cast", both(M * N),
             lambda: mx.mx_quantize_dim0_dim1(dY, buf["dyq"], buf["dys"], buf["dytq"], buf["dyts"])),
            g_dgrad, g_wgrad,
            n_w32, n_fwd,
            ("cast_dim0+dim1 dY'", "cast", both(M * NARROW),
             lambda: mx.mx_quantize_dim0_dim1(dYn, buf["dynq"], buf["dyns"], buf["dyntq"], buf["dynts"])),
            n_dgrad, n_wgrad,
        ]

    share_config = None
    if args.workload == "deepseek_share":
        assert not (unaligned or args.backward or args.separate_casts), \
            "--workload deepseek_share runs its own step; it takes none of the moe_g8 step's variants"
        del buf, X, W, dY, Wn, dYn
        torch.cuda.empty_cache()
        ops, share_config = deepseek_share_ops(mx, synth, to_dev, dev)

    if args.cycle_stamps:
        return cycle_stamps_main(args, ops, share_config)

    if args.only:
        # the casts an op depends on still run once, untimed, so its inputs exist
        for _, _, _, fn in ops:
            fn()
        torch.cuda.synchronize()
        sel = [o for o in ops if args.only in o[0]]
        assert sel, f"no op matches {args.only!r}"
        for _ in range(args.warmup + args.steps):
            for _, _, _, fn in sel:
                fn()
        torch.cuda.synchronize()
        print(json.dumps({"only": [o[0] for o in sel], "launches": args.warmup + args.steps}))
        return

    def step(events=None, only=None):
        for i, (_, _, _, fn) in enumerate(ops):
            rec = events is not None and (only is None or i == only)
            if rec:
                events[i][0].record()
            fn()
            if rec:
                events[i][1].record()

    def new_events(n):
        return [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in ops]
                for _ in range(n)]

    def mean_ms(evs, i):
        return float(np.mean([e[i][0].elapsed_time(e[i][1]) for e in evs]))

    def all_ms(evs, i):
        return [e[i][0].elapsed_time(e[i][1]) for e in evs]

    # W warm-up steps, with events around every launch: they pick the dominant
    # (longest) kernel; without warm-up, the op with the most work is taken
    wev = new_events(args.warmup)
    for w in range(args.warmup):
        step(wev[w])
    torch.cuda.synchronize()
    if args.warmup:
        dom_i = max(range(len(ops)), key=lambda i: mean_ms(wev[1:] or wev, i))
    else:
        dom_i = max(range(len(ops)), key=lambda i: ops[i][2] if ops[i][1] in PEAKS else 0)

    # timed region: exactly `steps` steps; events only around the dominant kernel's
    # launches (on the current stream, where every op runs), for its launch duration
    ev = new_events(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s], only=dom_i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    dom_ms = mean_ms(ev, dom_i)

    # per-kernel breakdown: a further `steps` steps with events around every launch
    # (reported only; not part of the timed region)
    bev = new_events(args.steps)
    for s in range(args.steps):
        step(bev[s])
    torch.cuda.synchronize()

    per_op = {}
    for i, (name, kind, units, _) in enumerate(ops):
        ms = dom_ms if i == dom_i else mean_ms(bev, i)
        mm = kind in PEAKS
        rate = units / (ms * 1e-3) / (1e12 if mm else 1e9)
        peak = PEAKS[kind] if mm else PEAK_HBM_GBPS
        each = all_ms(ev if i == dom_i else bev, i)
        per_op[name] = {"us": round(ms * 1e3, 2), ("tflops" if mm else "gbps"): round(rate, 1),
                        "frac": round(rate / peak, 4), "us_median": round(float(np.median(each)) * 1e3, 2),
                        "us_min": round(float(np.min(each)) * 1e3, 2)}

    gemm_flops = sum(u for _, k, u, _ in ops if k in PEAKS)
    cast_bytes = sum(u for _, k, u, _ in ops if k == "cast")
    gemm_us = sum(per_op[n]["us"] for n, k, _, _ in ops if k in PEAKS)
    cast_us = sum(per_op[n]["us"] for n, k, _, _ in ops if k == "cast")
    value = gemm_flops / (ms_per_step * 1e-3) / 1e12

    # practical HBM ceiling, measured after the timed region: a 1 GiB device-to-device
    # copy (2 GiB moved per copy), best of five
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    cps = []
    for _ in range(5):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        cps.append(c0.elapsed_time(c1))
    copy_gbps = round(2 * (1 << 30) / (min(cps) * 1e-3) / 1e9, 1)
    del src, dst
    # the same copy at each cast's own traffic (reads + writes = the cast's bytes), each
    # after a 512 MiB fill that leaves the caches holding dirty lines as the step's
    # GEMM outputs do, best of five: a smaller copy pays its ramp and tail on fewer bytes
    scrub = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
    copy_same = {}
    for name, kind, units, _ in ops:
        if kind != "cast":
            continue
        half = int(units // 2) // 16 * 16
        src = torch.empty(half, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        cps = []
        for r in range(5):
            scrub.fill_(r)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            dst.copy_(src)
            c1.record()
            torch.cuda.synchronize()
            cps.append(c0.elapsed_time(c1))
        gbps = 2 * half / (min(cps) * 1e-3) / 1e9
        copy_same[name] = {"copy_gbps": round(gbps, 1), "cast_frac_of_it": round(per_op[name]["gbps"] / gbps, 4)}
        del src, dst
    del scrub
    # practical MXFP8 ceiling, also after the timed region: the library's register-only
    # loop of the block-scaled MFMA on every SIMD (iters * 2^30 flops), best of three
    sink = mx.mx_probe_mfma(256)
    iters = 2048
    pts = []
    for _ in range(3):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        mx.mx_probe_mfma(iters, sink)
        c1.record()
        torch.cuda.synchronize()
        pts.append(c0.elapsed_time(c1))
    mfma_loop_tflops = round(iters * (1 << 30) / (min(pts) * 1e-3) / 1e12, 1)

    # dominant kernel: the longest launch of the step (timed inside the timed region)
    dom_name, dom_kind, dom_units, _ = ops[dom_i]
    dom = per_op[dom_name]
    achieved = dom_units / (dom["us"] * 1e-6) / 1e12
    traffic = (None if (unaligned or args.backward or args.precise) else
               load_traffic(("deepseek_share: " if share_config else "") + dom_name, dom_units))
    dom_peak = PEAKS[dom_kind]
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": dom_peak, "unit": "TFLOP/s",
                "frac": round(achieved / dom_peak, 4), "traffic": traffic, "kernel": dom_name,
                "flops_per_launch": dom_units, "avg_launch_us": dom["us"],
                # against the measured register-only MXFP8 loop (MXFP8 kernels only)
                "measured_ceiling": mfma_loop_tflops if dom_kind == "gemm" else None,
                "frac_of_measured_ceiling": round(achieved / mfma_loop_tflops, 4) if dom_kind == "gemm" else None}
    # the GEMMs' time at their own peaks over their measured time
    gemm_ideal_us = sum(u / (PEAKS[k] * 1e12) * 1e6 for _, k, u, _ in ops if k in PEAKS)

    cpu = None if (args.no_cpu_baseline or unaligned or args.backward or share_config or args.precise) \
        else cpu_baseline()
    workload = ("moe_g8 fwd+dgrad+wgrad: G=8 experts, M=16384 tokens, K=N=4096, "
                "grad_out 16384x4096, plus dense 576x4096 layer (32x32 weight scales, "
                "576-wide contraction in dgrad)")
    if args.backward:
        workload = (f"moe_g8 grouped step with the {args.backward} backward: G=8 experts, M=16384 tokens, "
                    f"K=N=4096; MXFP8 forward" + ("" if args.backward == "quantized" else
                                                  ", bf16 grouped dgrad and wgrad from "
                                                  + ("the saved bf16 operands" if args.backward == "high_precision"
                                                     else "the dequantized forward codes")) + " (no dense layer)")
    if args.precise:
        workload += ("; every GEMM from the same codes on the bf16 MFMA (both operands dequantized to bf16 "
                     "inside each op)")
    if unaligned:
        workload = (f"moe_g8 unaligned groups: G=8 experts, M=16384 tokens (per-row group sizes), K=N=4096; "
                    f"casts of X and dY padded to {Mg} rows in one pass, grouped fwd/dgrad/wgrad on padded "
                    f"offsets, Y and dX written unpadded (no dense layer)")

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 (MXFP8 codes dequantized to bf16, bf16 MFMA, fp32 accumulate)" if args.precise else
                  "mxfp8 (e4m3 x e4m3, e8m0 block scales, fp32 accumulate)" + (
                      "; bf16 backward GEMMs" if args.backward in ("high_precision", "dequantized") else "")),
        "data": "synthetic (seeded N(0,sigma) bf16, " + ("Zipf" if share_config else "multinomial")
                + " group sizes)",
        "config": share_config or {
            "workload": workload, "M": M, "K": K, "N": N, "G": G,
            "narrow": None if (unaligned or args.backward) else NARROW,
            "offs": offs_np.tolist(), "rows_padded": Mg if unaligned else None, "parallelism": "none (1 GPU)"},
        "gemm_tflops": round(gemm_flops / (gemm_us * 1e-6) / 1e12, 1),
        "gemm_frac_of_peak": round(gemm_ideal_us / gemm_us, 4),
        "cast_gbps": round(cast_bytes / (cast_us * 1e-6) / 1e9, 1),
        "cast_frac_of_hbm": round(cast_bytes / (cast_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "hbm_copy_gbps": copy_gbps,
        "mfma_loop_tflops": mfma_loop_tflops,
        "cast_frac_of_copy": round(cast_bytes / (cast_us * 1e-6) / 1e9 / copy_gbps, 4),
        "copy_same_bytes": copy_same,
        "step_gemm_gflop": round(gemm_flops / 1e9, 2), "step_cast_gb": round(cast_bytes / 1e9, 4),
        "roofline": roofline, "cpu_baseline": cpu, "kernels": per_op, "source_hash": src_hash(),
    }
    print(json.dumps(line), flush=True)


def stamp_summary(rec):
    """Per-block cycle records of one launch (rows of 8 words, see gemm.hip) -> summary.
    Cycles are shader-clock cycles (s_memtime) of each block's own compute unit."""
    rec = rec[rec[:, 7] == 1]
    if len(rec) == 0:
        return None
    t0, t1, t2, t3 = (rec[:, i].astype(np.float64) for i in range(4))
    hw = rec[:, 5].astype(np.uint64)
    n_iter = rec[:, 6].astype(np.float64)
    loop_ok = (t1 > 0) & (t2 >= t1) & (n_iter > 0)
    xcc = (hw >> np.uint64(32)).astype(np.int64)
    # compute unit: XCC, shader engine, shader array, CU (fields of HW_ID)
    cu = (xcc << 16) | (((hw >> np.uint64(13)) & np.uint64(7)).astype(np.int64) << 8) | \
         (((hw >> np.uint64(12)) & np.uint64(1)).astype(np.int64) << 4) | ((hw >> np.uint64(8)) & np.uint64(15)).astype(np.int64)
    spans, gaps, busy, by_xcd = [], [], 0.0, {}
    for c in np.unique(cu):
        idx = np.where(cu == c)[0]
        idx = idx[np.argsort(t0[idx])]
        span = t3[idx].max() - t0[idx].min()
        spans.append(span)
        busy += float(np.sum(t3[idx] - t0[idx]))
        gaps.extend((t0[idx][1:] - t3[idx][:-1]).tolist())
        by_xcd.setdefault(int(c >> 16), []).append(span)
    spans = np.array(spans)
    # tilings with two blocks per compute unit: blocks overlap, so neither the gap
    # between consecutive blocks nor a busy fraction is defined
    overlap = bool(gaps) and min(gaps) < 0
    per_step = (t2 - t1)[loop_ok] / n_iter[loop_ok]
    out = {
        "blocks": int(len(rec)), "compute_units": int(len(spans)), "k_steps_mean": round(float(n_iter.mean()), 2),
        "setup_cycles": round(float(np.mean((t1 - t0)[loop_ok])), 0) if loop_ok.any() else None,
        "loop_cycles": round(float(np.mean((t2 - t1)[loop_ok])), 0) if loop_ok.any() else None,
        "loop_cycles_per_k_step": round(float(per_step.mean()), 0) if loop_ok.any() else None,
        "epilogue_cycles": round(float(np.mean((t3 - t2)[loop_ok])), 0) if loop_ok.any() else None,
        "block_cycles": round(float(np.mean(t3 - t0)), 0),
        "gap_between_blocks_cycles": round(float(np.mean(gaps)), 0) if gaps and not overlap else None,
        "blocks_overlap_on_a_cu": overlap,
        "cu_span_cycles": {"mean": round(float(spans.mean()), 0), "min": round(float(spans.min()), 0),
                           "max": round(float(spans.max()), 0)},
        "busy_frac": None if overlap else round(busy / float(spans.sum()), 3),
        "per_xcd_span_mean_max": {str(x): [round(float(np.mean(v)), 0), round(float(np.max(v)), 0)]
                                  for x, v in sorted(by_xcd.items())},
    }
    if loop_ok.any():
        out["per_xcd_loop_cycles_per_k_step"] = {
            str(x): round(float(np.mean(per_step[xcc[loop_ok] == x])), 0) for x in sorted(set(xcc[loop_ok].tolist()))}
    return out


def cycle_stamps_main(args, ops, share_config):
    """Runs the step `warmup` times, then, in step order, every op once more, each GEMM
    alone between synchronisations, and prints each GEMM launch's per-block cycle
    breakdown (instrumented build: libmxfp8_stamps.so)."""
    import ctypes

    import torch

    from mxfp8_block_scaled_amd import _lib

    lib = _lib.load()
    lib.mx_cycle_stamps_blocks.restype = ctypes.c_int64
    lib.mx_cycle_stamps_read.argtypes = [ctypes.c_void_p]
    lib.mx_cycle_stamps_read.restype = ctypes.c_int
    lib.mx_cycle_stamps_clear.restype = ctypes.c_int
    nb = int(lib.mx_cycle_stamps_blocks())
    buf = np.zeros(nb * 8, dtype=np.uint64)
    for _ in range(args.warmup):
        for _, _, _, fn in ops:
            fn()
    torch.cuda.synchronize()
    res = {}
    for name, kind, _, fn in ops:
        if kind not in PEAKS:
            fn()
            continue
        torch.cuda.synchronize()
        assert lib.mx_cycle_stamps_clear() == 0
        fn()
        torch.cuda.synchronize()
        assert lib.mx_cycle_stamps_read(buf.ctypes.data) == 0
        rec = buf.reshape(nb, 8)
        launches = {"main": stamp_summary(rec[: nb // 2]), "quarter_tiles": stamp_summary(rec[nb // 2:])}
        res[name] = {k: v for k, v in launches.items() if v is not None}
    print(json.dumps({"cycle_stamps": res, "workload": share_config["workload"] if share_config else "moe_g8",
                      "warmup_steps": args.warmup, "source_hash": src_hash()}))


def host_facts():
    """The host the CPU baseline ran on: affine cores and CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"affine_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def blas_threads():
    import threadpoolctl

    return max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])


def linear_4096_main(args, mx, synth, to_dev, dev):
    import torch

    d = synth.linear_4096(0)
    X, W, dY = to_dev(d["x"]), to_dev(d["w"]), to_dev(d["dy"])
    Ml, Kl = X.shape
    Nl = W.shape[0]
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)  # noqa: E731
    sb = mx.mx_scale_bytes
    b = {"xq": u8(Ml, Kl), "xs": u8(sb(Ml, Kl)), "xtq": u8(Kl, Ml), "xts": u8(sb(Kl, Ml)),
         "wq": u8(Nl, Kl), "wqt": u8(Kl, Nl), "wsr": u8(sb(Nl, Kl)), "wsc": u8(sb(Kl, Nl)),
         "dyq": u8(Ml, Nl), "dys": u8(sb(Ml, Nl)), "dytq": u8(Nl, Ml), "dyts": u8(sb(Nl, Ml)),
         "y": bf(Ml, Nl), "dx": bf(Ml, Kl), "dw": bf(1, Nl, Kl)}
    ws = wgrad_workspace(mx, dev, 1, Ml, Nl, Kl)
    both = lambda n_elem: n_elem * BOTH_BYTES_PER_ELEM  # noqa: E731
    ops = [
        ("cast_dim0+dim1 X", "cast", both(Ml * Kl),
         lambda: mx.mx_quantize_dim0_dim1(X, b["xq"], b["xs"], b["xtq"], b["xts"])),
        ("cast_w32 W", "cast", Nl * Kl * W32_BYTES_PER_ELEM,
         lambda: mx.mx_quantize_weight_32x32(W, True, b["wq"], b["wqt"], b["wsr"], b["wsc"])),
        ("gemm_fwd dense", "gemm", 2 * Ml * Nl * Kl,
         lambda: mx.mx_grouped_mm_fwd(b["xq"], b["xs"], b["wq"], b["wsr"], None, Ml, Nl, Kl, out=b["y"])),
        ("cast_dim0+dim1 dY", "cast", both(Ml * Nl),
         lambda: mx.mx_quantize_dim0_dim1(dY, b["dyq"], b["dys"], b["dytq"], b["dyts"])),
        ("gemm_dgrad dense", "gemm", 2 * Ml * Nl * Kl,
         lambda: mx.mx_grouped_mm_dgrad(b["dyq"], b["dys"], b["wqt"], b["wsc"], None, Ml, Nl, Kl, out=b["dx"])),
        ("gemm_wgrad dense", "gemm", 2 * Ml * Nl * Kl,
         lambda: mx.mx_grouped_mm_wgrad(b["dytq"], b["dyts"], b["xtq"], b["xts"], None, Ml, Nl, Kl, out=b["dw"],
                                        out_dtype=mx.MX_OUT_BF16, workspace=ws)),
    ]
    stream = torch.cuda.current_stream()

    def run(events=None):
        for i, (_, _, _, fn) in enumerate(ops):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    # eager warm-up with events around every launch: per-kernel table and the dominant kernel
    ev_pairs = lambda: [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in ops]  # noqa: E731
    eager = [ev_pairs() for _ in range(max(args.warmup, 1))]
    for e in eager:
        run(e)
    torch.cuda.synchronize()
    op_ms = [float(np.median([e[i][0].elapsed_time(e[i][1]) for e in eager[1:] or eager])) for i in range(len(ops))]
    dom_i = max(range(len(ops)), key=lambda i: op_ms[i] if ops[i][1] in PEAKS else -1)

    # the step as a HIP graph of `steps` steps (events recorded inside a capture give no
    # timings, so the dominant kernel is timed by events around its eager launches
    # in `steps` eager steps right after the timed replay)
    reps = args.steps
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for r in range(reps):
            for _, _, _, fn in ops:
                fn()
    torch.cuda.synchronize()
    graph.replay()  # warm-up replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()  # the timed region: `steps` steps, back to back
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / reps
    after = [ev_pairs() for _ in range(reps)]
    for e in after:
        run(e)
    torch.cuda.synchronize()
    dom_ms = float(np.mean([e[dom_i][0].elapsed_time(e[dom_i][1]) for e in after]))

    # the 256^3 small linear: its casts and fp32 forward, replayed the same way
    sd = synth.linear_small(0)
    A, B = to_dev(sd["a"]), to_dev(sd["b"])
    sbuf = {"aq": u8(256, 256), "as": u8(sb(256, 256)), "bq": u8(256, 256), "bs": u8(sb(256, 256)),
            "y": torch.empty(256, 256, dtype=torch.float32, device=dev)}

    def small():
        mx.mx_quantize_dim0(A, sbuf["aq"], sbuf["as"])
        mx.mx_quantize_dim0(B, sbuf["bq"], sbuf["bs"])
        mx.mx_grouped_mm_fwd(sbuf["aq"], sbuf["as"], sbuf["bq"], sbuf["bs"], None, 256, 256, 256,
                             out_dtype=mx.MX_OUT_F32, out=sbuf["y"])

    small()
    torch.cuda.synchronize()
    sgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(sgraph, stream=side):
        for _ in range(100):
            small()
    sgraph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sgraph.replay()
    torch.cuda.synchronize()
    small_us = (time.perf_counter() - t1) * 1e6 / 100

    per_op = {}
    for i, (name, kind, units, _) in enumerate(ops):
        ms = dom_ms if i == dom_i else op_ms[i]
        mm = kind in PEAKS
        rate = units / (ms * 1e-3) / (1e12 if mm else 1e9)
        per_op[name] = {"us": round(ms * 1e3, 2), ("tflops" if mm else "gbps"): round(rate, 1),
                        "frac": round(rate / (PEAKS[kind] if mm else PEAK_HBM_GBPS), 4),
                        "timed": ("events around its eager launches, `steps` steps after the timed replay (mean)"
                                  if i == dom_i else "eager warm-up steps (median)")}
    gemm_flops = sum(u for _, k, u, _ in ops if k in PEAKS)
    dom_name, dom_kind, dom_units, _ = ops[dom_i]
    achieved = dom_units / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAKS[dom_kind], "unit": "TFLOP/s",
                "frac": round(achieved / PEAKS[dom_kind], 4), "traffic": load_traffic("linear_4096: " + dom_name,
                                                                                       dom_units),
                "kernel": dom_name, "flops_per_launch": dom_units, "avg_launch_us": round(dom_ms * 1e3, 2)}
    cpu = None if args.no_cpu_baseline else linear_cpu_baseline(synth)
    line = {
        "metric": METRIC, "value": round(gemm_flops / (ms_per_step * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": reps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8 (e4m3 x e4m3, e8m0 block scales, fp32 accumulate)",
        "data": "synthetic (seeded N(0,sigma) bf16)",
        "config": {"workload": "linear_4096 MXFP8Linear fwd+dgrad+wgrad: X 4096x2048, W 4096x2048 (32x32 weight "
                               "scales), dY 4096x4096; one HIP graph of `steps` steps, replayed",
                   "M": Ml, "N": Nl, "K": Kl, "parallelism": "none (1 GPU)"},
        "small_linear_256_us": round(small_us, 2),
        "small_linear_256": "dim0 casts of A, B [256, 256] (1% zero, 1% outlier blocks) + fwd fp32 out, one "
                            "iteration of a 100-iteration HIP graph",
        "roofline": roofline, "cpu_baseline": cpu, "kernels": per_op, "source_hash": src_hash(),
    }
    print(json.dumps(line), flush=True)


def linear_cpu_baseline(synth):
    """The oracle on the whole linear_4096 step: casts of X, W (32x32), dY and the
    float64 fwd, dgrad, wgrad."""
    from oracle import mx as orc

    d = synth.linear_4096(0)
    t0 = time.perf_counter()
    xq, xs = orc.quantize_dim0(d["x"])
    wq, wqt, wsr, wsc = orc.quantize_weight_32x32(d["w"])
    orc.mx_grouped_mm_fwd(xq, xs, wq, wsr, None, 1)
    dyq, dys = orc.quantize_dim0(d["dy"])
    orc.mx_grouped_mm_fwd(dyq, dys, wqt, wsc, None, 1)
    dytq, dyts = orc.quantize_dim1(d["dy"])
    xtq, xts = orc.quantize_dim1(d["x"])
    orc.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, None, 1)
    dt = time.perf_counter() - t0
    flops = 3 * 2 * 4096 * 4096 * 2048
    return dict({"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
                 "seconds": round(dt, 2),
                 "sample": "the whole step: oracle casts of X, W (32x32), dY and float64 fwd+dgrad+wgrad (numpy; "
                           "casts single-threaded, BLAS matmul on `cores` threads)"}, **host_facts())


def cpu_baseline():
    """The CPU oracle on a bounded slice of the same step, in the same unit.

    Slice: three experts, each a weight [4096, 4096] with 2048 token rows routed to
    it (and their grad_out rows), drawn like the benchmark's tensors: oracle dim0
    and dim1 casts of all three operands, then the float64 forward, dgrad and
    wgrad. About 10-15 s of host time. value = GEMM flops / total time.
    """
    from mxfp8_block_scaled_amd import synth
    from oracle import mx as orc

    experts, rows = 3, 2048
    r = synth.spawn(0, 3 * experts)
    data = [(synth.normal_bf16(r[3 * e], (rows, K), 1.0), synth.normal_bf16(r[3 * e + 1], (N, K), 0.02),
             synth.normal_bf16(r[3 * e + 2], (rows, N), 1e-2)) for e in range(experts)]
    t0 = time.perf_counter()
    for x, w, dy in data:
        xq, xs = orc.quantize_dim0(x)
        wq, ws = orc.quantize_dim0(w)
        orc.mx_grouped_mm_fwd(xq, xs, wq, ws, None, 1)
        dyq, dys = orc.quantize_dim0(dy)
        wtq, wts = orc.quantize_dim1(w)
        orc.mx_grouped_mm_fwd(dyq, dys, wtq, wts, None, 1)
        dytq, dyts = orc.quantize_dim1(dy)
        xtq, xts = orc.quantize_dim1(x)
        orc.mx_grouped_mm_wgrad(dytq, dyts, xtq, xts, None, 1)
    dt = time.perf_counter() - t0
    flops = experts * 3 * 2 * rows * N * K
    return dict({"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
                 "seconds": round(dt, 2),
                 "sample": f"{experts} expert slices, each {rows} token rows x W[{N},{K}]; oracle dim0+dim1 casts of "
                           "X, W, dY and float64 fwd+dgrad+wgrad (numpy; casts single-threaded, BLAS matmul on "
                           "`cores` threads)"}, **host_facts())


if __name__ == "__main__":
    main()
