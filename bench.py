#!/usr/bin/env python3
"""Benchmark of the NVFP4 hot path on one MI355X.

One step runs every stage of the path once over synthetic inputs resident in
HBM:
  quantize  the 8B-shaped layer set (q, k, v, o, gate, up, down; Student-t
            x 0.02, fp32): absmax with a computed tensor scale (amax pass +
            quantize pass), the absmax pass alone with that scale given,
            and the MSE scale search with that scale given;
  gemv      W4A16 decode: W [14336, 4096] and [4096, 14336], M = 1, 4, 16
            (weights rotated over enough copies to defeat the 256 MB MALL);
  gemm      W4A4 prefill: A [4096, 4096] bf16 with 1 % x20 outlier columns
            against gate and up [14336, 4096] (gate quantizes A, up reuses it);
            a Flux-like double-stream DiT block: image M = 4096 and text
            M = 512 tokens, to_q/k/v 3072x3072 (k, v reuse q's activation),
            MLP up 12288x3072 and down 3072x12288;
  lora      the same block with a fused rank-32 low-rank branch on q/k/v
            (one 9216x3072 layer), MLP up and MLP down, and again as
            SVDQuant layers (per-channel smoothing folded into the same pass)
            (reported per stage, outside value);
  calibrate the static activation scale: running amax and the FP8
            candidate sweep over four 512x3072 batches and the 4096x3072
            image-stream input, and the prefill gate product with a
            calibrated scale given (one-pass activation quantization);
            reported outside value.
Every stage is launched eagerly on torch's current stream (the stream the
library launches on) between two HIP events; before each stage a short GPU
spin kernel holds the queue so the host has enqueued the whole stage before
it starts, and the events time only GPU work (no host launch gaps).  The printed JSON line reports
value = mean over {quantize pass HBM %, GEMV HBM %, W4A4 GEMM MFMA %} of the
fraction of MI355X peak, plus per-stage numbers, the roofline of the
dominant kernel and the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK = 8.0e12           # bytes/s
MFMA16_PEAK = 2.5e15        # dense fp16/bf16 MFMA flop/s
VALU_PEAK = 256 * 64 * 2.4e9  # non-packed fp32/fp64 lane-ops/s: 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz
GEMV_COPIES = 16            # 16 x 33 MB = 529 MB, twice the 256 MB MALL (8 copies measured the same)
DIT_SUSTAINED_BLOCKS = 4    # DiT blocks run back to back in the sustained stage


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-peaks", action="store_true", help="skip the measured copy and bf16 GEMM reference rates")
    p.add_argument("--phases", default="quantize,gemv,gemm,lora,calibrate",
                   help="comma list of quantize, gemv, gemm (= prefill + dit), prefill, dit, lora "
                        "(the DiT block with a fused rank-32 LoRA), calibrate (static activation scale sweep and "
                        "the prefill gate with that scale); lora and calibrate are reported, not part of value")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a plain device-to-device copy of BYTES (HBM counter calibration) and exit")
    return p.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w4a4_prefill_traffic.json")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in ("gemm.hip", "device_common.hpp"):
        with open(os.path.join(ROOT, "dit_quantization_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


VALU_FILE = os.path.join(ROOT, "profiles", "quantize_mse_valu.json")


def mse_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in ("quantize_mse.hip", "device_common.hpp"):
        with open(os.path.join(ROOT, "dit_quantization_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_mse_lane_ops():
    """VALU lane-operations per element of the MSE search, counted with
    rocprofv3 (SQ_INSTS_VALU x 64 / elements) on the layer set, or None when
    the kernel source changed after the counters were taken."""
    try:
        with open(VALU_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != mse_source_hash():
        return None
    return d.get("lane_ops_per_element")


def stored_traffic():
    """HBM bytes per launch of the prefill GEMM kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs, or None when the kernel source
    changed after the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def e4m3_table():
    vals = [m / 8 * 2.0 ** -6 for m in range(8)]
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append((1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def mse_candidates(x, sg):
    """Number of scale candidates the MSE search visits per block (host count,
    used only to express the search's work against the ALU roofline)."""
    e4 = e4m3_table()
    amax = np.abs(x.reshape(-1, 16)).max(axis=1).astype(np.float64)
    a = amax / (6.0 * sg)
    lo = np.searchsorted(e4[1:], a / 2, side="left") + 1
    hi = np.searchsorted(e4[1:], np.minimum(2 * a, 448.0), side="right")
    return np.maximum(hi - lo + 1, 1).sum()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this library has no multi-GPU path "
              "(the products would shard column-parallel over weight rows, one process per GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    from dit_quantization_amd import inputs
    from dit_quantization_amd import nvfp4 as nv
    from dit_quantization_amd import svdquant

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration}), flush=True)
        return
    phases = set(args.phases.split(","))
    t0 = time.time()

    def f32(x):
        return torch.from_numpy(x).to(dev)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    stream = torch.cuda.current_stream()

    stages = {}   # name -> (stage function, calls, algorithmic bytes, flops, alu ops per run)

    def capture(name, fn, nbytes=0.0, flops=0.0, ops=0.0, calls=1):
        log(f"[stage] {name}: first run")
        fn()                                  # first run: loads code objects, checks the arguments
        torch.cuda.synchronize()
        stages[name] = (fn, calls, nbytes, flops, ops)

    # ------------------------------------------------------------ quantize
    layer_elems = 0
    mse_ops_source = None
    if "quantize" in phases:
        log("[setup] layer set")
        qbuf = []
        mse_ops = 0.0
        for name, w in inputs.layerset():
            xd = f32(w)
            rows, cols = w.shape
            out_a = (torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
                     torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev),
                     torch.empty(1, dtype=torch.float32, device=dev))
            out_m = (torch.empty_like(out_a[0]), torch.empty_like(out_a[1]), torch.empty_like(out_a[2]))
            out_f = (torch.empty_like(out_a[0]), torch.empty_like(out_a[1]), torch.empty_like(out_a[2]))
            ws = torch.empty(nv.workspace_bytes(nv.OP_QUANTIZE, rows, cols), dtype=torch.uint8, device=dev)
            nv.quantize_absmax(xd, workspace=ws, out=out_a)
            torch.cuda.synchronize()
            sg = float(out_a[2].item())
            out_m[2].fill_(sg)
            out_f[2].fill_(sg)
            qbuf.append((xd, out_a, out_m, out_f, ws, sg, rows, cols))
            layer_elems += rows * cols
            mse_ops += mse_candidates(w, sg) * 16 * 6.0
            del w
        n = layer_elems

        def q_dynamic():
            for xd, out_a, out_m, out_f, ws, sg, rows, cols in qbuf:
                nv.quantize_absmax(xd, workspace=ws, out=out_a)

        def q_pass():
            for xd, out_a, out_m, out_f, ws, sg, rows, cols in qbuf:
                nv.lib().nvfp4_quantize_absmax(nv._ptr(xd), nv.F32, rows, cols, nv._ptr(out_a[0]),
                                               nv._ptr(out_a[1]), nv._ptr(out_a[2]), nv.GLOBAL_GIVEN, None, 0,
                                               nv._stream())

        def q_mse():
            for xd, out_a, out_m, out_f, ws, sg, rows, cols in qbuf:
                nv.lib().nvfp4_quantize_mse(nv._ptr(xd), nv.F32, rows, cols, nv._ptr(out_m[0]), nv._ptr(out_m[1]),
                                            nv._ptr(out_m[2]), nv.GLOBAL_GIVEN, None, 0, nv._stream())

        def q_4o6():
            for xd, out_a, out_m, out_f, ws, sg, rows, cols in qbuf:
                nv.lib().nvfp4_quantize_4o6(nv._ptr(xd), nv.F32, rows, cols, nv._ptr(out_f[0]), nv._ptr(out_f[1]),
                                            nv._ptr(out_f[2]), nv.GLOBAL_GIVEN, None, 0, nv._stream())

        capture("quantize_absmax_dynamic", q_dynamic, nbytes=n * (4 + 4 + 0.5625))
        capture("quantize_absmax_pass", q_pass, nbytes=n * (4 + 0.5625))
        # ALU work of the MSE search: the counted lane-ops per element when
        # they were taken on this kernel source, else the op model
        counted = stored_mse_lane_ops()
        mse_ops_source = "rocprofv3 SQ_INSTS_VALU" if counted else "model: 6 ops per element and candidate"
        capture("quantize_mse", q_mse, nbytes=n * (4 + 0.5625), ops=counted * n if counted else mse_ops)
        # four-over-six: at most 2 candidates per block, 16 elements x 6 ops each
        capture("quantize_4o6", q_4o6, nbytes=n * (4 + 0.5625), ops=n / 16 * 2 * 16 * 6.0)

    # ------------------------------------------------------------ gemv
    if "gemv" in phases:
        log("[setup] gemv weights")
        for wi, w in enumerate(inputs.gemv_weights()):
            N, K = w.shape
            c, s, g = nv.quantize_absmax(f32(w))
            copies = [(c.clone(), s.clone()) for _ in range(GEMV_COPIES)]
            del c, s
            xb = bf16(inputs.gemv_x(K, 16))
            for M in (1, 4, 16):
                xm = xb[:M].contiguous()
                ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(GEMV_COPIES)]
                wsb = nv.workspace_bytes(nv.OP_GEMV_W4A16, M, N)   # split-K partials (M > 4, short weights)
                gws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None

                def run(copies=copies, xm=xm, ys=ys, g=g, gws=gws):
                    for (cc, ss), y in zip(copies, ys):
                        nv.gemv_w4a16(xm, cc, ss, g, out=y, workspace=gws, split_k=gws is not None)

                nbytes = GEMV_COPIES * (N * K * 0.5625 + 2 * M * K + 2 * M * N)
                capture(f"gemv_{N}x{K}_M{M}", run, nbytes=nbytes, flops=GEMV_COPIES * 2.0 * M * N * K,
                        calls=GEMV_COPIES)
            del w

    # ------------------------------------------------------------ gemm
    if "gemm" in phases or "prefill" in phases:
        log("[setup] prefill")
        a = bf16(inputs.prefill_activation())
        wts = {}
        for name, w in inputs.layerset(["gate", "up"]):
            wts[name] = nv.quantize_mse(f32(w))
            del w
        M, K = a.shape
        N = wts["gate"][0].shape[0]
        ws = torch.empty(nv.workspace_bytes(nv.OP_GEMM_W4A4, M, K), dtype=torch.uint8, device=dev)
        y_gate = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        y_up = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def prefill_gate():
            nv.gemm_w4a4(a, *wts["gate"], workspace=ws, out=y_gate)

        def prefill_up():
            nv.gemm_w4a4(a, *wts["up"], workspace=ws, out=y_up, reuse_act=True)

        capture("gemm_prefill_gate_actquant", prefill_gate, flops=2.0 * M * N * K,
                nbytes=M * K * (2 + 2 + 2 + 2) + N * K * 0.5625 + 2 * M * N)
        capture("gemm_prefill_up_reuse", prefill_up, flops=2.0 * M * N * K,
                nbytes=M * K * 2 + N * K * 0.5625 + 2 * M * N)

    # The image and text streams of a double-stream DiT block are independent
    # until the joint attention, which needs both streams' q, k and v; the
    # MLPs come after it.  A phase can run the two streams' products on two
    # HIP streams (both at the default priority), forked from and joined back
    # into the timed stream.  In the MLP phase the image MLP-up product fills
    # the chip, so the text MLP is queued behind it and runs beside the image
    # MLP-down product, whose 192 tiles leave a quarter of the CUs idle.
    side = torch.cuda.Stream()

    def two_streams(run_img, run_txt):
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            run_txt()
        run_img()
        main.wait_stream(side)

    def mlp_two_streams(img, txt):
        main = torch.cuda.current_stream()
        img[1]()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            txt[1]()
            txt[2]()
        img[2]()
        main.wait_stream(side)

    def dit_phases(img, txt):
        """img, txt: (q/k/v products, MLP up, MLP down) of one stream each."""
        two_streams(img[0], txt[0])
        mlp_two_streams(img, txt)

    if "gemm" in phases or "dit" in phases:
        log("[setup] dit block")
        a_img, a_txt, h_img, h_txt = inputs.dit_activations()
        dit_calls = []
        for stream_id, (aa, hh) in enumerate(((a_img, h_img), (a_txt, h_txt))):
            ad, hd = bf16(aa), bf16(hh)
            Ms = aa.shape[0]
            w = {name: nv.quantize_mse(f32(x)) for name, x in inputs.dit_weights(stream_id)}
            # workspaces with room for split-K partial sums (used by the short text-stream products)
            ws_a = torch.empty(max(nv.gemm_workspace_bytes(Ms, w[name][0].shape[0], ad.shape[1])
                                   for name in ("to_q", "to_k", "to_v", "mlp_up")), dtype=torch.uint8, device=dev)
            ws_h = torch.empty(nv.gemm_workspace_bytes(Ms, w["mlp_down"][0].shape[0], hd.shape[1]), dtype=torch.uint8,
                               device=dev)
            outs = {name: torch.empty((Ms, w[name][0].shape[0]), dtype=torch.bfloat16, device=dev) for name in w}
            dit_calls.append((ad, hd, w, ws_a, ws_h, outs))
        dit_flops = 0.0
        for ad, hd, w, ws_a, ws_h, outs in dit_calls:
            for name, (c, s, g) in w.items():
                dit_flops += 2.0 * ad.shape[0] * c.shape[0] * c.shape[1] * 2

        def dit_stream(ad, hd, w, ws_a, ws_h, outs):
            def qkv():
                nv.gemm_w4a4(ad, *w["to_q"], workspace=ws_a, out=outs["to_q"])
                nv.gemm_w4a4(ad, *w["to_k"], workspace=ws_a, out=outs["to_k"], reuse_act=True)
                nv.gemm_w4a4(ad, *w["to_v"], workspace=ws_a, out=outs["to_v"], reuse_act=True)

            def up():   # the MLP input is quantized anew
                nv.gemm_w4a4(ad, *w["mlp_up"], workspace=ws_a, out=outs["mlp_up"])

            def down():
                nv.gemm_w4a4(hd, *w["mlp_down"], workspace=ws_h, out=outs["mlp_down"])
            return qkv, up, down

        dit_img, dit_txt = dit_stream(*dit_calls[0]), dit_stream(*dit_calls[1])

        # Grouped launches (nvfp4_gemm_w4a4_group): one phase's image and text
        # products in one grid of 256x256 tiles, both activations quantized
        # first (k and v reuse q's quantized input).
        def group_phase(names, act):
            prods = []
            for ad, hd, w, ws_a, ws_h, outs in dit_calls:
                a_t, ws_t = (hd, ws_h) if act == "h" else (ad, ws_a)
                for j, name in enumerate(names):
                    prods.append({"a": a_t, "w": w[name], "workspace": ws_t, "out": outs[name], "reuse_act": j > 0})
            return prods

        grouped = [group_phase(["to_q", "to_k", "to_v"], "a"), group_phase(["mlp_up"], "a"),
                   group_phase(["mlp_down"], "h")]

        # The block: the six q/k/v products of both streams as one grouped
        # launch (648 tiles), then the MLPs on two HIP streams.
        def dit_block():
            nv.gemm_w4a4_group(grouped[0])
            mlp_two_streams(dit_img, dit_txt)

        capture("gemm_dit_block", dit_block, flops=dit_flops)

        # The linears of consecutive blocks / denoising steps back to back,
        # with no idle gap between blocks (reported beside the isolated block,
        # outside value).
        def dit_blocks_sustained():
            for _ in range(DIT_SUSTAINED_BLOCKS):
                dit_block()

        capture("dit_block_sustained", dit_blocks_sustained, flops=DIT_SUSTAINED_BLOCKS * dit_flops,
                calls=DIT_SUSTAINED_BLOCKS)

        # Two other schedules of the same products, reported beside it: every
        # phase on two HIP streams (q/k/v too), and every phase as one grouped
        # launch on one stream.
        def dit_block_two_streams():
            dit_phases(dit_img, dit_txt)

        capture("dit_block_two_streams", dit_block_two_streams, flops=dit_flops)

        def dit_block_grouped():
            for prods in grouped:
                nv.gemm_w4a4_group(prods)

        capture("dit_block_grouped", dit_block_grouped, flops=dit_flops)

    if "calibrate" in phases:
        # Static activation scale: running amax + FP8 candidate sweep over
        # calibration batches (four 512x3072 text-stream batches and the
        # 4096x3072 image-stream input), then the prefill gate product with
        # that scale given, whose activation quantization is one pass.
        log("[setup] calibration batches")
        cal = []
        for seed in range(4):
            x = inputs.normal_f32((512, 3072), 500 + seed)
            x, _ = inputs.with_outlier_columns(x, 30, 600 + seed)
            cal.append(bf16(inputs.to_bf16_bits(x)))
        cal.append(bf16(inputs.dit_activations()[0]))
        cal_blocks = sum(t.numel() for t in cal) / 16
        cal_ws = torch.empty(max(nv.workspace_bytes(nv.OP_ACT_CALIBRATE, *t.shape) for t in cal), dtype=torch.uint8,
                             device=dev)
        cal_amax = torch.zeros(1, dtype=torch.float32, device=dev)
        cal_err = torch.zeros(nv.SWEEP_CANDIDATES, dtype=torch.float64, device=dev)
        cal_scale = torch.empty(1, dtype=torch.float32, device=dev)

        def calibrate():
            cal_amax.zero_()
            cal_err.zero_()
            for t in cal:
                nv.act_amax(t, cal_amax, workspace=cal_ws)
            for t in cal:
                nv.act_scale_sweep(t, cal_amax, cal_err, cal_scale, workspace=cal_ws)

        capture("calibrate_sweep", calibrate, nbytes=cal_blocks * 16 * 2 * 2,
                ops=cal_blocks * nv.SWEEP_CANDIDATES * 16 * 6.0)

        a_pf = bf16(inputs.prefill_activation())
        (_, w_gate), = list(inputs.layerset(["gate"]))
        wq_gate = nv.quantize_mse(f32(w_gate))
        del w_gate
        Mp, Kp = a_pf.shape
        Np = wq_gate[0].shape[0]
        pf_scale, _, _ = nv.calibrate_act_scale([a_pf])
        ws_pf = torch.empty(nv.workspace_bytes(nv.OP_GEMM_W4A4, Mp, Kp), dtype=torch.uint8, device=dev)
        y_pf = torch.empty((Mp, Np), dtype=torch.bfloat16, device=dev)

        def static_gate():
            nv.gemm_w4a4(a_pf, *wq_gate, a_global=pf_scale, workspace=ws_pf, out=y_pf)

        capture("static_prefill_gate", static_gate, flops=2.0 * Mp * Np * Kp)

    if "lora" in phases:
        # The same block with a rank-32 low-rank branch fused into every
        # product: q/k/v as one [9216, 3072] layer sharing one branch, MLP up
        # and down each with their own; every call quantizes its input and
        # computes L = x down^T in the same pass.
        log("[setup] dit block with LoRA")
        a_img, a_txt, h_img, h_txt = inputs.dit_activations()
        lora_calls = []
        lora_flops = 0.0
        for stream_id, (aa, hh) in enumerate(((a_img, h_img), (a_txt, h_txt))):
            ad, hd = bf16(aa), bf16(hh)
            Ms = aa.shape[0]
            raw = dict(inputs.dit_weights(stream_id))
            layers = [("qkv", np.concatenate([raw["to_q"], raw["to_k"], raw["to_v"]]), ad),
                      ("mlp_up", raw["mlp_up"], ad), ("mlp_down", raw["mlp_down"], hd)]
            del raw
            for li, (name, wf, act) in enumerate(layers):
                N, K = wf.shape
                wq = nv.quantize_mse(f32(wf))
                down, up = (bf16(t) for t in inputs.lora_factors(32, K, N, 300 + 10 * stream_id + li))
                wsl = torch.empty(nv.workspace_bytes(nv.OP_GEMM_W4A4_LORA, Ms, K), dtype=torch.uint8, device=dev)
                out = torch.empty((Ms, N), dtype=torch.bfloat16, device=dev)
                # SVDQuant smoothing multipliers from this layer's channel ranges
                a_k = torch.zeros(K, dtype=torch.float32, device=dev)
                nv.channel_amax(act, a_k)
                _, smooth = svdquant.smoothing(a_k.cpu().numpy(), np.abs(wf).max(axis=0))
                lora_calls.append((act, wq, down, up, wsl, out, torch.from_numpy(smooth).to(dev)))
                lora_flops += 2.0 * Ms * N * K + 2.0 * Ms * 32 * (K + N)
            del layers

        n_img = len(lora_calls) // 2   # the image stream's layers come first

        def lora_layer(call, svdq):
            act, wq, down, up, wsl, out, smooth = call
            return lambda: nv.gemm_w4a4(act, *wq, workspace=wsl, out=out, lora=(down, up),
                                        smooth=smooth if svdq else None)

        def lora_stream(calls, svdq):   # (q/k/v, MLP up, MLP down) layers of one stream
            return tuple(lora_layer(c, svdq) for c in calls)

        lora_img, lora_txt = lora_stream(lora_calls[:n_img], False), lora_stream(lora_calls[n_img:], False)
        svdq_img, svdq_txt = lora_stream(lora_calls[:n_img], True), lora_stream(lora_calls[n_img:], True)

        def dit_block_lora():
            dit_phases(lora_img, lora_txt)

        def dit_block_svdq():
            dit_phases(svdq_img, svdq_txt)

        capture("lora_dit_block", dit_block_lora, flops=lora_flops)
        capture("svdq_dit_block", dit_block_svdq, flops=lora_flops)

    torch.cuda.synchronize()
    log(f"[setup] done in {time.time() - t0:.1f}s; stages: {list(stages)}")

    # ------------------------------------------------------------ timing
    names = list(stages)
    ev = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in names}
    acc = {k: 0.0 for k in names}
    step_start, step_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # GPU spin long enough for the host to enqueue any one stage behind it
    spin = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spin[0].record(stream)
    torch.cuda._sleep(1 << 20)
    spin[1].record(stream)
    torch.cuda.synchronize()
    cycles = int((1 << 20) * 2.0 / max(spin[0].elapsed_time(spin[1]), 1e-3))   # ~2 ms

    def one_step(record):
        for k in names:
            torch.cuda._sleep(cycles)
            if record:
                ev[k][0].record(stream)
            stages[k][0]()
            if record:
                ev[k][1].record(stream)

    log("[timing] warmup")
    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()
    total_ms = 0.0
    log("[timing] timed steps")
    for _ in range(args.steps):
        step_start.record(stream)
        one_step(True)
        step_end.record(stream)
        torch.cuda.synchronize()
        total_ms += step_start.elapsed_time(step_end)
        for k in names:
            acc[k] += ev[k][0].elapsed_time(ev[k][1])
    ms_per_step = sum(acc.values()) / args.steps     # GPU work per step (spins excluded)
    wall_ms_per_step = total_ms / args.steps
    per = {}
    for k in names:
        g, calls, nbytes, flops, ops = stages[k]
        t = acc[k] / args.steps / 1e3     # seconds per replay
        per[k] = {"us": t * 1e6, "us_per_call": t * 1e6 / calls}
        if nbytes:
            per[k]["GB_s"] = nbytes / t / 1e9
            per[k]["hbm_frac"] = nbytes / t / HBM_PEAK
        if flops:
            per[k]["TFLOP_s"] = flops / t / 1e12
            per[k]["mfma_frac"] = flops / t / MFMA16_PEAK
        if ops:
            per[k]["Gops_s"] = ops / t / 1e9
            per[k]["valu_frac"] = ops / t / VALU_PEAK
        log(f"  {k:32s} {json.dumps(per[k])}")

    comps = {}
    if "quantize_absmax_pass" in per:
        comps["quantize_hbm_frac"] = per["quantize_absmax_pass"]["hbm_frac"]
    gv = [k for k in per if k.startswith("gemv_")]
    if gv:
        tb = sum(stages[k][2] for k in gv)
        tt = sum(per[k]["us"] for k in gv) / 1e6
        comps["gemv_hbm_frac"] = tb / tt / HBM_PEAK
        comps["gemv_GB_s"] = tb / tt / 1e9
    gm = [k for k in per if k.startswith("gemm_")]
    if gm:
        tf = sum(stages[k][3] for k in gm)
        tt = sum(per[k]["us"] for k in gm) / 1e6
        comps["gemm_mfma_frac"] = tf / tt / MFMA16_PEAK
        comps["gemm_TFLOP_s"] = tf / tt / 1e12
    fracs = [comps[k] for k in ("quantize_hbm_frac", "gemv_hbm_frac", "gemm_mfma_frac") if k in comps]
    value = 100.0 * sum(fracs) / len(fracs) if fracs else 0.0

    # dominant kernel: the kernel family with the largest share of the step
    # time (stages grouped by the kernel that does their work), measured on
    # its representative single-launch stage
    family = {"quantize_mse": "mse", "quantize_4o6": "mse", "quantize_absmax_pass": "absmax",
              "quantize_absmax_dynamic": "absmax"}
    share = {}
    gemm_family = ("dit_block_sustained", "dit_block_two_streams", "dit_block_grouped", "lora_dit_block",
                   "svdq_dit_block", "static_prefill_gate")
    for k in names:
        f = family.get(k, "gemm" if k.startswith("gemm_") or k in gemm_family else "gemv" if k.startswith("gemv_")
                       else k)
        share[f] = share.get(f, 0.0) + per[k]["us"]
    representative = {"mse": "quantize_mse", "absmax": "quantize_absmax_pass", "gemm": "gemm_prefill_up_reuse"}
    top = max(share, key=share.get)
    dom = representative.get(top, top)
    roofline = None
    kernel_of = {
        "quantize_mse": ("quantize_mse_kernel", "alu"),
        "quantize_absmax_pass": ("quantize_absmax_kernel", "hbm"),
        "gemm_prefill_up_reuse": ("gemm_w4a4_kernel<256,256>", "mfma"),
    }
    if dom in kernel_of and dom in per:
        kname, bound = kernel_of[dom]
        g, calls, nbytes, flops, ops = stages[dom]
        t = per[dom]["us"] / 1e6
        if bound == "mfma":
            roofline = {"bound": "mfma", "kernel": kname, "achieved": flops / t / 1e12, "peak": 2500.0,
                        "unit": "TFLOP/s", "frac": flops / t / MFMA16_PEAK, "traffic": stored_traffic(),
                        "algorithmic_bytes": nbytes}
        elif bound == "alu":
            roofline = {"bound": "alu", "kernel": kname, "achieved": ops / t / 1e12, "peak": VALU_PEAK / 1e12,
                        "unit": "Tops/s", "frac": ops / t / VALU_PEAK, "traffic": None}
        else:
            roofline = {"bound": "hbm", "kernel": kname, "achieved": nbytes / t / 1e9, "peak": 8000.0,
                        "unit": "GB/s", "frac": nbytes / t / HBM_PEAK, "traffic": None}
        roofline["launch_us"] = per[dom]["us_per_call"] if calls == 1 else per[dom]["us"]

    peaks = None if args.no_peaks else measured_peaks(torch, dev)
    if roofline is not None:
        ref = None
        if peaks and roofline["bound"] == "mfma":
            ref = peaks["mfma_f16_loop_TFLOP_s"]
            roofline["frac_vs_vendor_bf16_gemm"] = roofline["achieved"] / peaks["bf16_gemm_TFLOP_s"]
        elif peaks and roofline["bound"] == "hbm":
            ref = peaks["hbm_read_1GiB_GB_s"]
        roofline["frac_vs_measured"] = roofline["achieved"] / ref if ref else None
        roofline["measured_peak"] = ref

    cpu = None if args.no_cpu_baseline else cpu_baseline(comps)

    line = {
        "metric": "quantize GB/s + W4A16 GEMV GB/s + W4A4 GEMM TFLOP/s, each as % of MI355X peak",
        "value": round(value, 3),
        "unit": "% of MI355X peak (mean of quantize-pass HBM, GEMV HBM, W4A4 GEMM MFMA fractions)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "wall_ms_per_step_incl_queue_spins": round(wall_ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 codes, e4m3 scales) -> f16/bf16 mfma, f32 accumulate",
        "data": "synthetic (seeded numpy PCG64; Student-t/Gaussian weights, outlier-channel activations)",
        "config": {"workload": "nvfp4 hot path: 8B layer-set quantize (absmax + MSE), decode GEMV "
                               "14336x4096 / 4096x14336 at M=1,4,16, W4A4 prefill 4096x4096x14336 (gate+up), "
                               "Flux-like double-stream DiT block (img 4096 + txt 512 tokens, hidden 3072)",
                   "layer_set_elements": layer_elems},
        "components": {k: round(v, 5) for k, v in comps.items()},
        "stages": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in per.items()},
        "roofline": roofline,
        "mse_ops_source": mse_ops_source if "quantize" in phases else None,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def measured_peaks(torch, dev):
    """Rates this GPU reaches on plain work, next to the datasheet peaks:
    - mfma_f16_loop_TFLOP_s: back-to-back v_mfma_f32_32x32x16_f16 with no
      memory traffic (the probe library), the matrix cores' ceiling at the
      running clock;
    - hbm_read_33MB_GB_s: one streaming read of a 33 MB buffer per launch
      (each workgroup one contiguous segment, the best of three grid sizes),
      rotating over 16 copies (529 MB, twice the MALL) like the decode GEMV's
      weights: the read ceiling at the GEMV's size (launch ramp included);
    - hbm_read_1GiB_GB_s: the same read over 1 GiB (best of two grids);
    - hbm_copy_GB_s: a 1 GiB device-to-device copy (read + write bytes);
    - bf16_gemm_TFLOP_s: a bf16 8192^3 product through torch (the vendor
      GEMM library).
    Each is the best of several launches timed with HIP events on torch's
    current stream (the stream the probes launch on)."""
    import ctypes
    out = {}
    probes = ctypes.CDLL(os.path.join(ROOT, "dit_quantization_amd", "libnvfp4_probes.so"))
    probes.probe_mfma_f16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    probes.probe_mfma_f16_flops.restype = ctypes.c_double
    probes.probe_mfma_f16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    probes.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def best_of(fn, reps=5):
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 1e3
            best = t if best is None else min(best, t)
        return best

    blocks, iters = 256 * 8, 2048
    mout = torch.empty(blocks * 256, dtype=torch.float32, device=dev)

    def mfma():
        if probes.probe_mfma_f16(ctypes.c_void_p(mout.data_ptr()), blocks, iters, sp) != 0:
            raise RuntimeError("probe_mfma_f16 launch failed")

    mfma()
    out["mfma_f16_loop_TFLOP_s"] = probes.probe_mfma_f16_flops(blocks, iters) / best_of(mfma) / 1e12
    del mout
    rout = torch.empty(1 << 14, dtype=torch.int32, device=dev)
    gemv_bytes = 14336 * 4096 * 9 // 16            # 33,030,144 B: one decode weight (codes + scales)
    copies = [torch.empty(gemv_bytes, dtype=torch.uint8, device=dev) for _ in range(GEMV_COPIES)]

    def reader(bufs, nbytes, blocks):
        def run():
            for c in bufs:
                probes.probe_read(ctypes.c_void_p(c.data_ptr()), nbytes, ctypes.c_void_p(rout.data_ptr()), blocks, sp)
        return run

    best = 0.0
    for blocks in (1024, 2048, 4096):              # workgroups of 256 lanes, one contiguous segment each
        run = reader(copies, gemv_bytes, blocks)
        run()
        best = max(best, GEMV_COPIES * gemv_bytes / best_of(run) / 1e9)
    out["hbm_read_33MB_GB_s"] = best
    del copies
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    best = 0.0
    for blocks in (2048, 8192):
        run = reader([src], n, blocks)
        run()
        best = max(best, n / best_of(run) / 1e9)
    out["hbm_read_1GiB_GB_s"] = best
    dst = torch.empty_like(src)
    out["hbm_copy_GB_s"] = 2.0 * n / best_of(lambda: dst.copy_(src)) / 1e9
    del src, dst, rout
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    c = a @ b
    out["bf16_gemm_TFLOP_s"] = 2.0 * 8192 ** 3 / best_of(lambda: torch.matmul(a, b, out=c)) / 1e12
    del a, b, c
    torch.cuda.synchronize()
    return {k: round(v, 1) for k, v in out.items()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(gpu_comps):
    """The CPU oracle (plain C, fp64, OpenMP over blocks/pairs) on a bounded
    sample of the same workloads, expressed in the same unit: once on every
    core the process may run on, once on one thread."""
    import oracle
    from dit_quantization_amd import inputs
    cores = len(os.sched_getaffinity(0))
    (_, w), = list(inputs.layerset(["q"]))
    w1 = inputs.normal_f32((4096, 4096), 1, 0.02)
    c, s, sg = oracle.quantize(w1, threads=cores)
    x = inputs.bf16_bits_to_f32(inputs.gemv_x(4096, 1))
    a = inputs.bf16_bits_to_f32(inputs.prefill_activation()[:128])

    def sample(threads):
        res = {}
        # quantize (absmax with its amax pass) on the layer set's q tensor (2^24 elements)
        t = time.perf_counter()
        oracle.quantize(w, oracle.ABSMAX, threads=threads)
        dt = time.perf_counter() - t
        qfrac = w.size * (4 + 4 + 0.5625) / dt / HBM_PEAK
        res["quantize_GB_s"] = w.size * (4 + 4 + 0.5625) / dt / 1e9
        # MSE on 2^20 elements
        xm = w[:256]
        t = time.perf_counter()
        oracle.quantize(xm, oracle.MSE, threads=threads)
        res["mse_GB_s"] = xm.size * (4 + 0.5625) / (time.perf_counter() - t) / 1e9
        # GEMV: M = 1 against a 4096 x 4096 weight
        t = time.perf_counter()
        oracle.dot_w4a16(x, c, s, sg, threads=threads)
        dt = time.perf_counter() - t
        gbytes = 4096 * 4096 * 0.5625 + 2 * 4096 + 2 * 4096
        gfrac = gbytes / dt / HBM_PEAK
        res["gemv_GB_s"] = gbytes / dt / 1e9
        # W4A4: 128 x 1024 outputs of the prefill product (K = 4096), activation quantization included
        t = time.perf_counter()
        ac, as_, asg = oracle.quantize(a, threads=threads)
        oracle.dot_w4a4(ac, as_, asg, c[:1024], s[:1024], sg, 4096, threads=threads)
        dt = time.perf_counter() - t
        flops = 2.0 * 128 * 1024 * 4096
        mfrac = flops / dt / MFMA16_PEAK
        res["gemm_GFLOP_s"] = flops / dt / 1e9
        return 100.0 * (qfrac + gfrac + mfrac) / 3, {k: round(v, 4) for k, v in res.items()}

    t0 = time.perf_counter()
    value, comps = sample(cores)
    t_all = time.perf_counter() - t0
    t0 = time.perf_counter()
    value1, comps1 = sample(1)
    t_one = time.perf_counter() - t0
    return {"value": value, "unit": "% of MI355X peak (same formula as value)", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "absmax quantize of the 4096x4096 fp32 q tensor (with amax), MSE of 256x4096, "
                      "W4A16 M=1 x 4096x4096 weight, W4A4 128x1024 outputs of the prefill product (K=4096, "
                      "activation quantization included)",
            "components": comps, "sample_seconds": round(t_all, 2),
            "single_thread": {"value": value1, "cores": 1, "components": comps1, "sample_seconds": round(t_one, 2)}}


if __name__ == "__main__":
    main()
