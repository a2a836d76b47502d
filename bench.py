"""Benchmark of the QAM-W codec hot path on one MI355X.

Workload (the configuration the headline metric is quoted on): one attention-projection-shaped
weight matrix W of 4096 x 4096 bf16 (Student-t(5) x 0.015, 41 outlier columns x 10, channel scale
s_j = |N(0,1)|^0.5 + 0.1), Hadamard block 128, K = 2048 codebook (11-bit pair index) trained by 20
Lloyd iterations on 2^20 unit-circular-Gaussian points.

One step = encode (pair calibration over the first 1024 rows + encode of all rows) followed by
decode to BF16, with W, the codes and the output already in HBM.  Steps rotate over enough
copies of the buffers (>= 1 GiB) that the 256 MiB last-level cache cannot serve repeats.
The codebook training and the search-index build depend on the codebook only; they run and
are timed once in the same run and reported beside the step.

Beside the step: the fused dequantize-and-multiply of section 1 (y = x W^T from the codes, M = 1,
4, 16 activation rows) against hipBLASLt on the decoded BF16 W and against decode-then-multiply; the
reconstruction error of joint 2D, polar and scalar (d = 1) coding at equal bits on the same matrix;
the activation-aware channel scale (time on a 2048-row calibration batch, and the layer-output error
it leaves for several alpha);
and the polar baseline of section 3.5 (5 + 6 and 4 + 4 bits) on the same matrix:
codebook build, encode, encoder kernel alone, decode.

After the step, unless --no-stack: a 40-layer 13B-shaped stack (per layer q, k, v, o 5120x5120,
gate and up 13824x5120, down 5120x13824; 12.7 G weights, bf16 Student-t(4) x 0.015 drawn on the
GPU) is encoded and then decoded to BF16 in HBM, all 280 matrices back to back, for the
sustained rates.

Prints one JSON line.  --gpus N with N > 1 is not supported (single-GPU build).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encode Mweights/s + decode GB/s (BF16 out), 4096×4096 W, K=2048 codebook"
HBM_PEAK_GBPS = 8000.0
# 256 CUs x 4 SIMD x 16 lanes x 2.4 GHz: one 32/64-bit VALU lane operation per lane per clock
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--rot-gib", type=float, default=1.25, help="bytes of rotated buffers")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 40-layer 13B-shaped stack (sustained encode and decode)")
    return ap.parse_args()


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key, src_files, per_launch_alg_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        k = d["kernels"][kernel_key]
        if k.get("source_hash") != source_hash(src_files):
            return None
        return k["hbm_bytes_per_dispatch"]
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth_inputs as synth
    import weight_quantization_codec_amd as q

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q.load()
    cfg = synth.config(1)
    m = cfg.matrices[0]
    d_out, d_in, block, bits = m.d_out, m.d_in, cfg.block, cfg.bits[0]
    n_w = d_out * d_in

    # ---------------------------------------------------------------- inputs (host -> HBM, untimed)
    w_host = m.weights()
    s_host = m.channel_scale()
    sign = q.DEFAULT_SIGN_SEED   # seed of the rotation's sign mask
    pts_host = synth.points(cfg.seed, synth.SID_POINTS, cfg.n_points)
    w0 = torch.from_numpy(w_host.view(np.int16)).view(torch.bfloat16).to(dev)
    scale = torch.from_numpy(s_host).to(dev)
    pts = torch.from_numpy(pts_host).to(dev)

    # plain copy of known size: calibrates the FETCH_SIZE / WRITE_SIZE counters in profiled runs
    cp_src = torch.ones((128 << 20,), dtype=torch.float32, device=dev)   # 512 MiB read, 512 MiB written
    cp_dst = torch.empty_like(cp_src)
    torch.mul(cp_src, 1.0, out=cp_dst)
    torch.cuda.synchronize()
    del cp_src, cp_dst

    # ---------------------------------------------------------------- codebook + index (timed once)
    stream = torch.cuda.current_stream()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record(stream)
    cb, trace = q.codebook_train(pts, bits, cfg.lloyd_iters)
    e1.record(stream)
    index = q.codebook_index(cb, bits)
    e2.record(stream)
    torch.cuda.synchronize()
    train_ms, index_ms = e0.elapsed_time(e1), e1.elapsed_time(e2)
    mse = float(trace[-1].item()) / 2**32 / cfg.n_points

    # ---------------------------------------------------------------- rotated buffers
    stride = q.row_stride(d_in, bits)
    per_set = n_w * 2 + d_out * stride + n_w * 2 + d_out * 2
    n_sets = max(2, int(math.ceil(args.rot_gib * (1 << 30) / per_set)))
    sets = []
    for _ in range(n_sets):
        sets.append({
            "w": w0.clone(),
            "codes": torch.empty((d_out, stride), dtype=torch.uint8, device=dev),
            "norm": torch.empty((d_out,), dtype=torch.int16, device=dev),
            "sigma": torch.empty((d_in // 2,), dtype=torch.float32, device=dev),
            "out": torch.empty((d_out, d_in), dtype=torch.bfloat16, device=dev),
        })
    ws = torch.empty((q.encode_workspace(d_out, d_in, bits),), dtype=torch.uint8, device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev)

    def enc(bset, sigma=None):
        q.encode(bset["w"], cb, bits, index, scale=scale, sign_seed=sign, block=block, sigma=sigma, status=status,
                 workspace=ws, out={"codes": bset["codes"], "norm": bset["norm"], "sigma": bset["sigma"]})

    def dec(bset):
        q.decode(bset["codes"], bset["norm"], bset["sigma"], cb, bits, d_in, scale=scale, sign_seed=sign,
                 block=block, out=bset["out"])

    def step(i):
        bset = sets[i % n_sets]
        enc(bset)
        dec(bset)

    # ---------------------------------------------------------------- warmup + timed steps
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = n_w * args.steps / elapsed / 1e6
    assert int(status.item()) == 0, "data-fault flags raised: %d" % int(status.item())

    # ---------------------------------------------------------------- per-kernel timing (HIP events)
    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n   # ms per call

    n_k = max(args.steps, 50)
    sigma_fixed = sets[0]["sigma"].clone()
    enc_full_ms = timed(lambda i: enc(sets[i % n_sets]), n_k)
    enc_kernel_ms = timed(lambda i: enc(sets[i % n_sets], sigma=sigma_fixed), n_k)  # k_encode alone
    dec_ms = timed(lambda i: dec(sets[i % n_sets]), n_k)                          # k_decode alone

    # algorithmic bytes per weight (B-bit pair index = B/16 bytes per weight, f16 norm per row)
    code_b = bits / 16.0 + 2.0 / d_in
    dec_bytes = n_w * (code_b + 2.0)
    enc_bytes = n_w * (2.0 + code_b)
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    # algorithmic lane operations per weight of the encoder: scale (1), square-accumulate (2),
    # log2(b) butterflies, pair scaling (1), fp32 rounding (1), one fp32 distance evaluation per
    # pair (6 per pair = 3), packing (1 per pair = 0.5)
    L = int(round(math.log2(block)))
    enc_ops_per_w = 1 + 2 + L + 1 + 1 + 3 + 0.5
    enc_tops = n_w * enc_ops_per_w / (enc_kernel_ms * 1e-3) / 1e12

    src_enc = ["weight_quantization_codec_amd/csrc/k_encode.hip", "weight_quantization_codec_amd/csrc/qamw_device.hpp"]
    src_dec = ["weight_quantization_codec_amd/csrc/k_decode.hip", "weight_quantization_codec_amd/csrc/qamw_device.hpp"]
    roof_enc = {"bound": "alu", "kernel": "k_encode", "achieved": round(enc_tops, 3), "peak": round(VALU_PEAK_TOPS, 2),
                "unit": "Tops/s", "frac": round(enc_tops / VALU_PEAK_TOPS, 4),
                "traffic": traffic_from_profile("k_encode", src_enc, enc_bytes),
                "alg_ops_per_weight": enc_ops_per_w, "launch_ms": round(enc_kernel_ms, 5),
                "hbm_GBps": round(enc_bytes / (enc_kernel_ms * 1e-3) / 1e9, 1)}
    roof_dec = {"bound": "hbm", "kernel": "k_decode", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                "traffic": traffic_from_profile("k_decode", src_dec, dec_bytes),
                "alg_bytes_per_launch": int(dec_bytes), "launch_ms": round(dec_ms, 5)}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "Mweights/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "attn-4096x4096 bf16 Student-t(5)x0.015, 41 outlier cols x10, b=128, K=2048 (B=11)",
                   "d_out": d_out, "d_in": d_in, "block": block, "bits": bits, "rotated_sets": n_sets},
        "encode_Mweights_per_s": round(n_w / (enc_full_ms * 1e-3) / 1e6, 1),
        "decode_GB_per_s": round(dec_gbps, 1),
        "decode_Mweights_per_s": round(n_w / (dec_ms * 1e-3) / 1e6, 1),
        "encode_ms": round(enc_full_ms, 5), "decode_ms": round(dec_ms, 5),
        "train_ms": round(train_ms, 3), "index_ms": round(index_ms, 4), "lloyd_final_mse": round(mse, 7),
        "bpw": round(q.row_stride(d_in, bits) * 8 / d_in + 16.0 / d_in, 4),
        "roofline": roof_enc, "roofline_decode": roof_dec,
    }

    # ---------------------------------------------------------------- fused dequantize-and-multiply (section 1)
    result["qgemm"] = qgemm_run(torch, q, sets, n_sets, cb, bits, scale, sign, block, timed)

    # ---------------------------------------------------------------- polar baseline (section 3.5)
    for ba, bp in ((5, 6), (4, 4)):
        result["polar_%d_%d" % (ba, bp)] = polar_run(torch, q, sets, n_sets, scale, sign, block, ba, bp, timed, stream)

    # ---------------------------------------------------------------- activation-aware channel scale
    result["act_scale"] = act_scale_run(torch, q, sets[0], cb, bits, index, sign, block, timed)

    # ---------------------------------------------------------------- d = 2 vs polar vs d = 1 at equal bits
    result["ablation"] = ablation_run(torch, q, sets[0], pts, cfg, cb, bits, scale, sign, block)

    # ---------------------------------------------------------------- 40-layer stack (sustained rates)
    if not args.no_stack:
        del sets
        torch.cuda.empty_cache()
        result["stack40"] = stack_run(torch, q, cb, index, bits, block, stream)

    # ---------------------------------------------------------------- CPU oracle baseline (whole workload)
    if not args.no_cpu:
        import oracle
        orc = oracle.get()
        cb_h = cb.cpu().numpy()
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        t0 = time.perf_counter()
        sb_host = orc.sign_mask(sign, d_in)
        sig, _ = orc.calibrate(w_host[:1024], s_host, sb_host, block)
        e = orc.encode(w_host, s_host, sb_host, block, cb_h, bits, sig, want_idx=False)
        orc.decode(e["codes"], e["norm"], d_in, sig, cb_h, bits, s_host, sb_host, block)
        t_cpu = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(n_w / t_cpu / 1e6, 3), "unit": "Mweights/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": "whole 4096x4096 round trip (calibrate 1024 rows, encode, decode), "
                                            "%.1f s" % t_cpu}
    print(json.dumps(result), flush=True)


def qgemm_run(torch, q, sets, n_sets, cb, bits, scale, sign, block, timed):
    """y = x W^T for M activation rows with W in its codes (qamw_qgemm), against hipBLASLt on the
    decoded BF16 W (torch.matmul) and against decode-then-multiply, on the step's matrix; the code
    and weight buffers rotate over the step's sets."""
    dev = sets[0]["w"].device
    d_out, d_in = sets[0]["w"].shape
    for i in range(n_sets):   # every set holds the codes and the BF16 decode of the same matrix
        q.decode(sets[i]["codes"], sets[i]["norm"], sets[i]["sigma"], cb, bits, d_in, scale=scale, sign_seed=sign,
                 block=block, out=sets[i]["out"])
    stride = q.row_stride(d_in, bits)
    res = {}
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    for M in (1, 4, 16):
        x = torch.randn((M, d_in), device=dev, generator=g).to(torch.bfloat16)
        y = torch.empty((M, d_out), dtype=torch.float32, device=dev)
        ws = torch.empty((q.qgemm_workspace(M, d_out, d_in),), dtype=torch.uint8, device=dev)
        tmp = torch.empty((d_out, d_in), dtype=torch.bfloat16, device=dev)

        def fused(i):
            b = sets[i % n_sets]
            q.qgemm(x, b["codes"], b["norm"], b["sigma"], cb, bits, scale=scale, sign_seed=sign, block=block, out=y,
                    workspace=ws)

        def bf16(i):
            torch.matmul(x, sets[i % n_sets]["out"].t())

        def dec_mm(i):
            b = sets[i % n_sets]
            q.decode(b["codes"], b["norm"], b["sigma"], cb, bits, d_in, scale=scale, sign_seed=sign, block=block, out=tmp)
            torch.matmul(x, tmp.t())

        for fn in (fused, bf16, dec_mm):   # first calls pick and load library kernels
            for i in range(10):
                fn(i)
        torch.cuda.synchronize()
        t_f, t_b, t_d = timed(fused, 200), timed(bf16, 200), timed(dec_mm, 100)
        alg = d_out * stride + d_out * 2 + M * d_in * 2 + M * d_out * 4   # codes, norms, x, y
        res["M%d" % M] = {"qgemm_us": round(t_f * 1e3, 2), "bf16_matmul_us": round(t_b * 1e3, 2),
                          "decode_then_matmul_us": round(t_d * 1e3, 2),
                          "speedup_vs_bf16": round(t_b / t_f, 3), "speedup_vs_decode_matmul": round(t_d / t_f, 3),
                          "hbm_GBps": round(alg / (t_f * 1e-3) / 1e9, 1),
                          "hbm_frac": round(alg / (t_f * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "kernel": "vector units" if M < 6 else "matrix cores (fp32)"}
        del ws, tmp
    return res


def act_scale_run(torch, q, bset, cb, bits, index, sign, block, timed):
    """qamw_act_scale on a 2048 x d_in BF16 calibration batch (time, HBM rate), and the layer-output
    error ||X dW^T||_F^2 / ||X W^T||_F^2 of the step's matrix coded with s = r^alpha for several
    alpha (alpha = 0 is s = 1).  Activations: synthetic, drawn on the GPU, per-channel RMS
    exp(0.5 N(0,1)) with 1% of the channels x30 (the strong channels of LLM activations)."""
    w = bset["w"]
    d_out, d_in = w.shape
    dev = w.device
    g = torch.Generator(device=dev)
    g.manual_seed(17)
    T = 2048
    rho = torch.exp(0.5 * torch.randn(d_in, device=dev, generator=g))
    strong = torch.randperm(d_in, device=dev, generator=g)[: d_in // 100]
    rho[strong] *= 30
    x = (torch.randn((T, d_in), device=dev, generator=g) * rho).to(torch.bfloat16)
    ws = torch.empty((q.load().qamw_act_scale_workspace(T, d_in),), dtype=torch.uint8, device=dev)
    for _ in range(5):
        q.act_scale(x, 0.3, workspace=ws)
    torch.cuda.synchronize()
    t_ms = timed(lambda i: q.act_scale(x, 0.3, workspace=ws), 100)
    res = {"T": T, "d_in": d_in, "act_scale_us": round(t_ms * 1e3, 2),
           "hbm_GBps": round(T * d_in * 2 / (t_ms * 1e-3) / 1e9, 1),
           "hbm_frac": round(T * d_in * 2 / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    xf = x.float()
    wf = w.float()
    y2 = float(torch.sum((xf @ wf.t()) ** 2))
    out = torch.empty((d_out, d_in), dtype=torch.float32, device=dev)
    errs = {}
    for alpha in (0.0, 0.3, 0.5):
        s = q.act_scale(x, alpha, workspace=ws)
        e = q.encode(w, cb, bits, index, scale=s, sign_seed=sign, block=block)
        q.decode(e["codes"], e["norm"], e["sigma"], cb, bits, d_in, scale=s, sign_seed=sign, block=block, out=out)
        errs["alpha_%g" % alpha] = round(float(torch.sum((xf @ (out - wf).t()) ** 2)) / y2, 7)
    res["output_error"] = errs
    res["data"] = "synthetic activations drawn on the GPU; relative layer-output error, lower is better"
    return res


def ablation_run(torch, q, bset, pts, cfg, cb11, bits11, scale, sign, block):
    """Relative reconstruction error ||W^ - W||_F / ||W||_F of the step's matrix (BF16 decode) for the
    joint 2D code (QAM-W), the polar code (section 3.5) and the scalar d = 1 code (section 2) at
    equal bits per pair; each is one GPU encode and decode.  QAM-W codebooks at B = 8 and 12 are
    trained like the step's (same points and iteration count)."""
    w = bset["w"]
    d_out, d_in = w.shape
    wf = w.float()
    wn = float(torch.linalg.vector_norm(wf))
    out = torch.empty_like(w)

    def err(table, nbits, index=None, thr=None, ba=None):
        if thr is None:
            idx = q.codebook_index(table, nbits) if index is None else index
            e = q.encode(w, table, nbits, idx, scale=scale, sign_seed=sign, block=block)
        else:
            e = q.encode_polar(w, ba, nbits - ba, thr, scale=scale, sign_seed=sign, block=block)
        q.decode(e["codes"], e["norm"], e["sigma"], table, nbits, d_in, scale=scale, sign_seed=sign, block=block,
                 out=out)
        return round(float(torch.linalg.vector_norm(out.float() - wf)) / wn, 6)

    res = {}
    for B in (8, 11, 12):
        row = {}
        if B == bits11:
            row["qamw_2d"] = err(cb11, B)
        else:
            cbB, _ = q.codebook_train(pts, B, cfg.lloyd_iters)
            row["qamw_2d"] = err(cbB, B)
        # the same training run longer: Lloyd from the first K points is far from converged after
        # the workload's iterations at these K
        cbL, trL = q.codebook_train(pts, B, 10 * cfg.lloyd_iters)
        row["qamw_2d_%dit" % (10 * cfg.lloyd_iters)] = err(cbL, B)
        row["lloyd_mse_%dit" % (10 * cfg.lloyd_iters)] = round(float(trL[-1].item()) / 2**32 / pts.shape[0], 7)
        ba = {8: 4, 11: 5, 12: 6}[B]
        _, thr, table = q.polar_codebook(ba, B - ba)
        row["polar_%d+%d" % (ba, B - ba)] = err(table, B, thr=thr, ba=ba)
        if B % 2 == 0:
            _, _, tab1 = q.scalar_codebook(B // 2)
            row["scalar_d1_%d+%d" % (B // 2, B // 2)] = err(tab1, B)
        res["B%d" % B] = row
    res["note"] = "relative Frobenius error of the BF16 decode of the step's synthetic matrix; lower is better"
    return res


def polar_run(torch, q, sets, n_sets, scale, sign, block, ba, bp, timed, stream):
    """The polar baseline on the step's workload: codebook build (once), encode with calibration,
    the encoder kernel alone (fixed sigma) and the decode of its codes with the product table."""
    dev = sets[0]["w"].device
    d_out, d_in = sets[0]["w"].shape
    n_w = d_out * d_in
    bits = ba + bp
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    levels, thr, table = q.polar_codebook(ba, bp)
    b.record(stream)
    torch.cuda.synchronize()
    cb_ms = a.elapsed_time(b)
    stride = q.row_stride(d_in, bits)
    codes = [torch.empty((d_out, stride), dtype=torch.uint8, device=dev) for _ in range(n_sets)]
    ws = torch.empty((q.encode_workspace(d_out, d_in, bits),), dtype=torch.uint8, device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev)

    def enc(i, sigma=None):
        bset = sets[i % n_sets]
        q.encode_polar(bset["w"], ba, bp, thr, scale=scale, sign_seed=sign, block=block, sigma=sigma, status=status,
                       workspace=ws, out={"codes": codes[i % n_sets], "norm": bset["norm"], "sigma": bset["sigma"]})

    def dec(i):
        bset = sets[i % n_sets]
        q.decode(codes[i % n_sets], bset["norm"], bset["sigma"], table, bits, d_in, scale=scale, sign_seed=sign,
                 block=block, out=bset["out"])

    for i in range(n_sets):
        enc(i)
        dec(i)
    n_k = 100
    enc_ms = timed(enc, n_k)
    sigma_fixed = sets[0]["sigma"].clone()
    enc_kernel_ms = timed(lambda i: enc(i, sigma_fixed), n_k)
    dec_ms = timed(dec, n_k)
    assert int(status.item()) == 0, "data-fault flags raised: %d" % int(status.item())
    dec_bytes = n_w * (bits / 16.0 + 2.0 / d_in + 2.0)
    out = {"ba": ba, "bp": bp, "codebook_ms": round(cb_ms, 4), "encode_ms": round(enc_ms, 5),
           "encode_Mweights_per_s": round(n_w / (enc_ms * 1e-3) / 1e6, 1),
           "encode_kernel_ms": round(enc_kernel_ms, 5), "decode_ms": round(dec_ms, 5),
           "decode_GB_per_s": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
           "bpw": round(stride * 8 / d_in + 16.0 / d_in, 4)}
    del codes
    return out


def stack_run(torch, q, cb, index, bits, block, stream):
    """Encode, then decode, the 280 matrices of a 40-layer 13B-shaped stack back to back."""
    dev = cb.device
    import synth_inputs as synth
    mats = []
    for spec in synth.config(4).matrices:   # per-layer seeds, drawn on the GPU (synth_gpu.hip)
        d_out, d_in = spec.d_out, spec.d_in
        stride = q.row_stride(d_in, bits)
        mats.append({"w": spec.weights_device(dev), "s": torch.from_numpy(spec.channel_scale()).to(dev), "d_in": d_in,
                     "codes": torch.empty((d_out, stride), dtype=torch.uint8, device=dev),
                     "norm": torch.empty((d_out,), dtype=torch.int16, device=dev),
                     "sigma": torch.empty((d_in // 2,), dtype=torch.float32, device=dev),
                     "out": torch.empty((d_out, d_in), dtype=torch.bfloat16, device=dev)})
    ws = torch.empty((max(q.encode_workspace(m["w"].shape[0], m["d_in"], bits) for m in mats),), dtype=torch.uint8,
                     device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def enc_all():
        for m in mats:
            q.encode(m["w"], cb, bits, index, scale=m["s"], sign_seed=q.DEFAULT_SIGN_SEED, block=block, status=status,
                     workspace=ws, out={"codes": m["codes"], "norm": m["norm"], "sigma": m["sigma"]})

    def dec_all():
        for m in mats:
            q.decode(m["codes"], m["norm"], m["sigma"], cb, bits, m["d_in"], scale=m["s"], sign_seed=q.DEFAULT_SIGN_SEED,
                     block=block, out=m["out"])

    def best_ms(fn, reps=3):
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b)
            best = t if best is None else min(best, t)
        return best

    enc_all()
    dec_all()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "data-fault flags raised in the stack: %d" % int(status.item())
    enc_ms = best_ms(enc_all)
    dec_ms = best_ms(dec_all)
    n_w = sum(m["w"].numel() for m in mats)
    dec_bytes = sum(m["codes"].numel() + m["norm"].numel() * 2 + m["out"].numel() * 2 for m in mats)
    res = {"matrices": len(mats), "weights": n_w, "encode_ms": round(enc_ms, 3),
           "encode_Mweights_per_s": round(n_w / (enc_ms * 1e-3) / 1e6, 1), "decode_ms": round(dec_ms, 3),
           "decode_GB_per_s": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
           "decode_frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "resident_GB": round((n_w * 2 + sum(m["codes"].numel() for m in mats) + n_w * 2) / 1e9, 1),
           "data": "synthetic, the seeded 40-layer workload drawn on the GPU; K=2048 codebook and b=128 of the step"}
    del mats
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
