"""Benchmark of the QAM-W codec hot path on one MI355X.

Workload of the headline line (the configuration the metric is quoted on): one attention-projection-
shaped weight matrix W of 4096 x 4096 bf16 (Student-t(5) x 0.015, 41 outlier columns x 10, channel
scale s_j = |N(0,1)|^0.5 + 0.1), Hadamard block 128, K = 2048 codebook (11-bit pair index) trained by
20 Lloyd iterations on 2^20 unit-circular-Gaussian points.

One step = encode (pair calibration over the first 1024 rows + encode of all rows) followed by
decode to BF16, with W, the codes and the output already in HBM.  Steps rotate over enough
copies of the buffers (>= 1 GiB) that the 256 MiB last-level cache cannot serve repeats.  `value`
is weights per second of whole steps (wall clock around K steps, synchronized on both sides).

Also in the line (every rate a median of 5 repeats, each at least 100 ms, timed with HIP events
on the stream the kernels run on, over >= 1 GiB of rotated buffers unless the workload is larger):
  peaks       plain copy (read + write) and fill (write only) of 1 GiB: the rates HBM gives
              kernels that only move bytes, beside the 8 TB/s published peak;
  configs     every workload: 256 x 512 fp32 (K = 256, b = 64, sigma 1/8: launch-bound); the
              step's 4096 x 4096; the 7B MLP pair (11008 x 4096 and 4096 x 11008, b = 256) with its
              codebook retrained by 50 Lloyd iterations on 2^22 points (evaluations per second);
              one 13B-shaped layer at 11 and 7 bits (K = 2048 and K = 128); the 40-layer stack
              (12.7 G weights) encoded end to end and decoded back to back, per matrix and grouped
              (qamw_decode_many);
  roofline    the step's dominant kernel (the encoder, VALU-bound) and the decoder (HBM-bound):
              achieved rate from the live timing, the published peak, and HBM traffic per launch
              from the committed rocprofv3 counters when they match the current sources;
  studies     the fused dequantize-and-multiply, the polar and scalar baselines, the
              activation-aware scale (skipped with --no-extras);
  cpu_baseline the CPU oracle on a bounded sample of the step's workload (all host threads and
              one thread), plus samples of the other workloads.

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
# 256 CUs x 4 SIMD16 x 16 lanes x 2.4 GHz: one 32- or 64-bit VALU lane operation per lane per clock
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# VALU lane operations per weight of the encoder by the hot-path analysis of the method: fp64
# front end (scale, norm, transform, pair scaling) about 14, the pruned nearest-codeword search
# about 6 per candidate over the wavefront's longest list (8-12 candidates per pair), packing 2:
# about 50 in all
ENC_ALG_OPS_PER_W = 50.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--rot-gib", type=float, default=1.25, help="bytes of rotated buffers")
    ap.add_argument("--no-stack", action="store_true", help="skip the 40-layer stack")
    ap.add_argument("--no-configs", action="store_true", help="only the step's workload")
    ap.add_argument("--no-extras", action="store_true", help="skip the fused product and baseline studies")
    return ap.parse_args()


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


ENC_SOURCES = ["weight_quantization_codec_amd/csrc/k_encode.hip", "weight_quantization_codec_amd/csrc/qamw_device.hpp"]
DEC_SOURCES = ["weight_quantization_codec_amd/csrc/k_decode128.hip", "weight_quantization_codec_amd/csrc/qamw_device.hpp",
               "weight_quantization_codec_amd/csrc/qamw_launch.hpp"]


def profile_entry(kernel_key, src_files):
    """The committed rocprofv3 counter summary of a kernel (profiles/counters.json), if it was
    taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        k = json.load(open(path))["kernels"][kernel_key]
        return k if k.get("source_hash") == source_hash(src_files) else None
    except (KeyError, ValueError):
        return None


class Timer:
    """Median per-call milliseconds of fn(i) over 5 repeats of at least min_ms each, timed with
    HIP events on `stream` (the stream the library's kernels are queued on)."""

    def __init__(self, torch, stream, min_ms=100.0, reps=5):
        self.torch, self.stream, self.min_ms, self.reps = torch, stream, min_ms, reps

    def __call__(self, fn, n_min=1):
        torch = self.torch
        ev = lambda: torch.cuda.Event(enable_timing=True)
        fn(0)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(self.stream)
        fn(1)
        b.record(self.stream)
        torch.cuda.synchronize()
        one = max(a.elapsed_time(b), 1e-3)
        n = max(n_min, int(math.ceil(self.min_ms / one)))
        res = []
        for _ in range(self.reps):
            a, b = ev(), ev()
            a.record(self.stream)
            for i in range(n):
                fn(i)
            b.record(self.stream)
            torch.cuda.synchronize()
            res.append(a.elapsed_time(b) / n)
        return float(np.median(res))


def n_rotated(bytes_per_set, gib):
    return max(2, int(math.ceil(gib * (1 << 30) / bytes_per_set)))


def peaks_run(torch, dev, timed):
    """Copy (read + write) and fill (write only) of 1 GiB of bf16."""
    n = (1 << 30) // 2
    x = torch.empty(n, dtype=torch.bfloat16, device=dev).uniform_()
    y = torch.empty_like(x)
    t_copy = timed(lambda i: y.copy_(x))
    t_fill = timed(lambda i: y.fill_(1.5))
    del x, y
    torch.cuda.empty_cache()
    return {"copy_GBps": round(2 * n * 2 / (t_copy * 1e-3) / 1e9, 1), "fill_GBps": round(n * 2 / (t_fill * 1e-3) / 1e9, 1),
            "bytes": 2 * n, "note": "torch copy_ and fill_ of 1 GiB bf16; copy counts bytes read plus written"}


def dec_bytes_of(d_out, d_in, bits, out_elem=2):
    """Algorithmic decode bytes: packed codes (bits/16 per weight), f16 norms, BF16 output."""
    return d_out * d_in * (bits / 16.0) + d_out * 2 + d_out * d_in * out_elem


def enc_bytes_of(d_out, d_in, bits, in_elem=2, calibrate=True):
    """Algorithmic encode bytes: W read once (plus the calibration re-read of min(1024, d_out) rows),
    packed codes and f16 norms written."""
    cal = min(1024, d_out) * d_in * in_elem if calibrate else 0
    return d_out * d_in * in_elem + cal + d_out * d_in * (bits / 16.0) + d_out * 2


def matrix_codec(torch, q, w_list, scale_list, cb, bits, index, block, timed, rot_gib, sigma_fixed=None):
    """Encode and decode timings of a list of matrices (one call each, back to back), over rotated
    copies of the inputs and outputs when they are smaller than rot_gib."""
    dev = cb.device
    per_set = sum(w.numel() * w.element_size() * 2 + w.shape[0] * (q.row_stride(w.shape[1], bits) + 2) for w in w_list)
    n_sets = n_rotated(per_set, rot_gib) if per_set < rot_gib * (1 << 30) else 1
    sets = []
    for k in range(n_sets):
        mats = []
        for w, s in zip(w_list, scale_list):
            d_out, d_in = w.shape
            mats.append({"w": w if k == 0 else w.clone(), "s": s, "d_in": d_in,
                         "codes": torch.empty((d_out, q.row_stride(d_in, bits)), dtype=torch.uint8, device=dev),
                         "norm": torch.empty((d_out,), dtype=torch.int16, device=dev),
                         "sigma": torch.empty((d_in // 2,), dtype=torch.float32, device=dev),
                         "out": torch.empty((d_out, d_in), dtype=torch.bfloat16, device=dev)})
        sets.append(mats)
    ws = torch.empty((max(q.encode_workspace(w.shape[0], w.shape[1], bits) for w in w_list),), dtype=torch.uint8,
                     device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev)

    def enc(i):
        for m in sets[i % n_sets]:
            q.encode(m["w"], cb, bits, index, scale=m["s"], block=block, sigma=sigma_fixed, status=status, workspace=ws,
                     out={"codes": m["codes"], "norm": m["norm"], "sigma": m["sigma"]})

    def dec(i):
        for m in sets[i % n_sets]:
            q.decode(m["codes"], m["norm"], m["sigma"] if sigma_fixed is None else sigma_fixed, cb, bits, m["d_in"],
                     scale=m["s"], block=block, out=m["out"])

    for i in range(n_sets):
        enc(i)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "data-fault flags raised: %d" % int(status.item())
    t_enc, t_dec = timed(enc), timed(dec)
    n_w = sum(w.numel() for w in w_list)
    in_elem = w_list[0].element_size()
    eb = sum(enc_bytes_of(w.shape[0], w.shape[1], bits, in_elem, sigma_fixed is None) for w in w_list)
    db = sum(dec_bytes_of(w.shape[0], w.shape[1], bits) for w in w_list)
    res = {"encode_us": round(t_enc * 1e3, 2), "encode_Mweights_per_s": round(n_w / (t_enc * 1e-3) / 1e6, 1),
           "encode_GBps": round(eb / (t_enc * 1e-3) / 1e9, 1),
           "decode_us": round(t_dec * 1e3, 2), "decode_GBps": round(db / (t_dec * 1e-3) / 1e9, 1),
           "decode_frac_of_8TBps": round(db / (t_dec * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "rotated_sets": n_sets}
    return res, sets


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
    stream = torch.cuda.current_stream()
    timed = Timer(torch, stream)

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

    # ---------------------------------------------------------------- HBM peaks of plain copies
    peaks = peaks_run(torch, dev, timed)

    # ---------------------------------------------------------------- codebook + index (per codebook)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record(stream)
    cb, trace = q.codebook_train(pts, bits, cfg.lloyd_iters)
    e1.record(stream)
    index = q.codebook_index(cb, bits)
    e2.record(stream)
    torch.cuda.synchronize()
    train_ms, index_ms = e0.elapsed_time(e1), e1.elapsed_time(e2)
    mse = float(trace[-1].item()) / 2**32 / cfg.n_points

    # ---------------------------------------------------------------- rotated buffers of the step
    stride = q.row_stride(d_in, bits)
    per_set = n_w * 2 + d_out * stride + n_w * 2 + d_out * 2
    n_sets = n_rotated(per_set, args.rot_gib)
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
    sigma_fixed = sets[0]["sigma"].clone()
    step_ms = timed(step)
    enc_full_ms = timed(lambda i: enc(sets[i % n_sets]))
    enc_kernel_ms = timed(lambda i: enc(sets[i % n_sets], sigma=sigma_fixed))   # the encoder kernel alone
    dec_ms = timed(lambda i: dec(sets[i % n_sets]))                              # the decoder kernel alone
    dec_bytes = dec_bytes_of(d_out, d_in, bits)
    enc_bytes = enc_bytes_of(d_out, d_in, bits, 2, calibrate=False)
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    enc_tops = n_w * ENC_ALG_OPS_PER_W / (enc_kernel_ms * 1e-3) / 1e12

    def traffic(entry):
        return None if entry is None else entry["hbm_bytes_per_dispatch"]

    pe, pd = profile_entry("k_encode", ENC_SOURCES), profile_entry("k_decode128", DEC_SOURCES)
    roof_enc = {"bound": "alu", "kernel": "k_encode<7,1024,bf16>", "achieved": round(enc_tops, 3),
                "peak": round(VALU_PEAK_TOPS, 2), "unit": "Tops/s", "frac": round(enc_tops / VALU_PEAK_TOPS, 4),
                "traffic": traffic(pe), "alg_ops_per_weight": ENC_ALG_OPS_PER_W,
                "alg_bytes_per_launch": int(enc_bytes), "launch_us": round(enc_kernel_ms * 1e3, 2),
                "hbm_GBps": round(enc_bytes / (enc_kernel_ms * 1e-3) / 1e9, 1),
                "valu_insts_per_weight": None if pe is None else pe.get("valu_lane_insts_per_weight"),
                "valu_busy": None if pe is None else pe.get("valu_busy")}
    roof_dec = {"bound": "hbm", "kernel": "k_decode128<11,bf16>", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                "frac_of_copy_peak": round(dec_gbps / peaks["copy_GBps"], 4), "traffic": traffic(pd),
                "alg_bytes_per_launch": int(dec_bytes), "launch_us": round(dec_ms * 1e3, 2)}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "Mweights/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "attn-4096x4096 bf16 Student-t(5)x0.015, 41 outlier cols x10, b=128, K=2048 (B=11)",
                   "d_out": d_out, "d_in": d_in, "block": block, "bits": bits, "rotated_sets": n_sets},
        "encode_Mweights_per_s": round(n_w / (enc_full_ms * 1e-3) / 1e6, 1),
        "decode_GB_per_s": round(dec_gbps, 1),
        "decode_Mweights_per_s": round(n_w / (dec_ms * 1e-3) / 1e6, 1),
        "step_us_events": round(step_ms * 1e3, 2), "encode_us": round(enc_full_ms * 1e3, 2),
        "encode_kernel_us": round(enc_kernel_ms * 1e3, 2), "decode_us": round(dec_ms * 1e3, 2),
        "train_ms": round(train_ms, 3), "index_ms": round(index_ms, 4), "lloyd_final_mse": round(mse, 7),
        "bpw": round(q.row_stride(d_in, bits) * 8 / d_in + 16.0 / d_in, 4),
        "peaks": peaks, "roofline": roof_enc, "roofline_decode": roof_dec,
    }

    # ---------------------------------------------------------------- studies on the step's matrix
    if not args.no_extras:
        result["qgemm"] = qgemm_run(torch, q, sets, n_sets, cb, bits, scale, sign, block, timed)
        for ba, bp in ((5, 6), (4, 4)):
            result["polar_%d_%d" % (ba, bp)] = polar_run(torch, q, sets, n_sets, scale, sign, block, ba, bp, timed,
                                                         stream)
        result["act_scale"] = act_scale_run(torch, q, sets[0], cb, bits, index, sign, block, timed)
        result["qgemm_13b_layer"] = qgemm13b_run(torch, q, synth, cb, index, bits, block, timed, args.rot_gib)
        result["ablation"] = ablation_run(torch, q, sets[0], pts, cfg, cb, bits, scale, sign, block)
    del sets, ws
    torch.cuda.empty_cache()

    # ---------------------------------------------------------------- the other workloads
    if not args.no_configs:
        result["configs"] = configs_run(torch, q, synth, timed, args.rot_gib, cb, index, peaks)
    if not args.no_stack:
        result["stack40"] = stack_run(torch, q, synth, cb, index, bits, block, timed, peaks)

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(synth, w_host, s_host, sign, block, cb.cpu().numpy(), bits)
    print(json.dumps(result), flush=True)


def configs_run(torch, q, synth, timed, rot_gib, cb1, index1, peaks):
    """Per-workload encode / decode rates (the step's own is in the main line)."""
    dev = cb1.device
    out = {}
    # 256 x 512 fp32, K = 256 from 2^16 points, b = 64, sigma fixed at 1/8: launch-bound
    c0 = synth.config(0)
    m0 = c0.matrices[0]
    pts0 = torch.from_numpy(synth.points(c0.seed, synth.SID_POINTS, c0.n_points)).to(dev)
    cb0, _ = q.codebook_train(pts0, c0.bits[0], c0.lloyd_iters)
    ix0 = q.codebook_index(cb0, c0.bits[0])
    w0 = torch.from_numpy(m0.weights()).to(dev)
    s0 = torch.from_numpy(m0.channel_scale()).to(dev)
    sig0 = torch.full((m0.d_in // 2,), c0.fixed_sigma, dtype=torch.float32, device=dev)
    r, _ = matrix_codec(torch, q, [w0], [s0], cb0, c0.bits[0], ix0, c0.block, timed, 0.0, sigma_fixed=sig0)
    r["note"] = "fp32 W, sigma given (1/8): one launch each, warm (the whole problem is 1 MB)"
    out[c0.name] = r

    # 7B MLP pair, b = 256, K = 2048 retrained by 50 Lloyd iterations on 2^22 points
    c2 = synth.config(2)
    pts2 = torch.from_numpy(synth.points(c2.seed, synth.SID_POINTS, c2.n_points)).to(dev)
    K = 1 << c2.bits[0]
    holder = {}

    def train(i):
        holder["cb"], holder["tr"] = q.codebook_train(pts2, c2.bits[0], c2.lloyd_iters)

    t_train = timed(train)
    cb2 = holder["cb"]
    ix2 = q.codebook_index(cb2, c2.bits[0])
    evals = float(c2.n_points) * K * c2.lloyd_iters
    r2 = {"lloyd": {"points": c2.n_points, "K": K, "iters": c2.lloyd_iters, "ms": round(t_train, 3),
                    "evals_per_s": round(evals / (t_train * 1e-3), 1),
                    "final_mse": round(float(holder["tr"][-1].item()) / 2**32 / c2.n_points, 7)}}
    for mm in c2.matrices:
        w = mm.weights_device(dev)
        s = torch.from_numpy(mm.channel_scale()).to(dev)
        r, sets = matrix_codec(torch, q, [w], [s], cb2, c2.bits[0], ix2, c2.block, timed, rot_gib)
        r["shape"] = [mm.d_out, mm.d_in]
        r2[mm.name] = r
        del sets, w
        torch.cuda.empty_cache()
    out[c2.name] = r2

    # one 13B-shaped layer at 11 bits (K = 2048) and 7 bits (K = 128), b = 128
    c3 = synth.config(3)
    pts3 = torch.from_numpy(synth.points(c3.seed, synth.SID_POINTS, c3.n_points)).to(dev)
    pts3b = torch.from_numpy(synth.points(c3.seed, c3.extra["k128_sid"], c3.extra["k128_points"])).to(dev)
    ws3 = [mm.weights_device(dev) for mm in c3.matrices]
    ss3 = [torch.from_numpy(mm.channel_scale()).to(dev) for mm in c3.matrices]
    r3 = {}
    for B, p in ((11, pts3), (7, pts3b)):
        cbB, _ = q.codebook_train(p, B, c3.lloyd_iters)
        ixB = q.codebook_index(cbB, B)
        r, sets = matrix_codec(torch, q, ws3, ss3, cbB, B, ixB, c3.block, timed, rot_gib)
        mats = sets[0]
        plan = q.DecodeManyPlan([{"codes": mt["codes"], "norm": mt["norm"], "sigma": mt["sigma"], "scale": mt["s"],
                                  "d_in": mt["d_in"], "out": mt["out"]} for mt in mats], cbB, B, block=c3.block)
        t_many = timed(lambda i: plan())
        db = sum(dec_bytes_of(mt["w"].shape[0], mt["d_in"], B) for mt in mats)
        r["decode_many_us"] = round(t_many * 1e3, 2)
        r["decode_many_GBps"] = round(db / (t_many * 1e-3) / 1e9, 1)
        r["decode_many_frac_of_8TBps"] = round(db / (t_many * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        r["bpw_d5120"] = round(q.row_stride(5120, B) * 8 / 5120 + 16.0 / 5120, 4)
        r3["B%d" % B] = r
        del sets, mats, plan
        torch.cuda.empty_cache()
    r3["note"] = "q, k, v, o 5120x5120, gate and up 13824x5120, down 5120x13824 back to back (one call each)"
    out[c3.name] = r3
    del ws3, ss3
    torch.cuda.empty_cache()
    return out


def stack_run(torch, q, synth, cb, index, bits, block, timed, peaks):
    """Encode, then decode, the 280 matrices of a 40-layer 13B-shaped stack back to back: one call per
    matrix, and the decode also as one grouped call (qamw_decode_many)."""
    dev = cb.device
    mats = []
    for spec in synth.config(4).matrices:   # per-layer seeds, drawn on the GPU
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

    def enc_all(i):
        for m in mats:
            q.encode(m["w"], cb, bits, index, scale=m["s"], sign_seed=q.DEFAULT_SIGN_SEED, block=block, status=status,
                     workspace=ws, out={"codes": m["codes"], "norm": m["norm"], "sigma": m["sigma"]})

    def dec_all(i):
        for m in mats:
            q.decode(m["codes"], m["norm"], m["sigma"], cb, bits, m["d_in"], scale=m["s"], sign_seed=q.DEFAULT_SIGN_SEED,
                     block=block, out=m["out"])

    plan = q.DecodeManyPlan([{"codes": m["codes"], "norm": m["norm"], "sigma": m["sigma"], "scale": m["s"],
                              "d_in": m["d_in"], "out": m["out"]} for m in mats], cb, bits, block=block)
    enc_all(0)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "data-fault flags raised in the stack: %d" % int(status.item())
    enc_ms = timed(enc_all)
    dec_ms = timed(dec_all)
    many_ms = timed(lambda i: plan())
    n_w = sum(m["w"].numel() for m in mats)
    dec_bytes = sum(dec_bytes_of(m["w"].shape[0], m["d_in"], bits) for m in mats)
    enc_bytes = sum(enc_bytes_of(m["w"].shape[0], m["d_in"], bits) for m in mats)
    gbps = lambda ms: dec_bytes / (ms * 1e-3) / 1e9
    res = {"matrices": len(mats), "weights": n_w,
           "encode_ms": round(enc_ms, 3), "encode_Mweights_per_s": round(n_w / (enc_ms * 1e-3) / 1e6, 1),
           "encode_GBps": round(enc_bytes / (enc_ms * 1e-3) / 1e9, 1),
           "decode_ms": round(dec_ms, 3), "decode_GB_per_s": round(gbps(dec_ms), 1),
           "decode_frac": round(gbps(dec_ms) / HBM_PEAK_GBPS, 4),
           "decode_many_ms": round(many_ms, 3), "decode_many_GB_per_s": round(gbps(many_ms), 1),
           "decode_many_frac": round(gbps(many_ms) / HBM_PEAK_GBPS, 4),
           "decode_many_frac_of_copy_peak": round(gbps(many_ms) / peaks["copy_GBps"], 4),
           "decode_many_frac_of_fill_peak": round(gbps(many_ms) / peaks["fill_GBps"], 4),
           "alg_decode_bytes": int(dec_bytes),
           "resident_GB": round((n_w * 2 + sum(m["codes"].numel() for m in mats) + n_w * 2) / 1e9, 1),
           "data": "synthetic, the seeded 40-layer workload drawn on the GPU; K=2048 codebook and b=128 of the step"}
    del mats, plan
    torch.cuda.empty_cache()
    return res


def cpu_baseline(synth, w_host, s_host, sign, block, cb_h, bits):
    """The CPU oracle (plain fp64 reference, never tuned) on bounded samples: the whole step's
    workload with every host thread (three runs), a quarter of it with one thread (extrapolated),
    and one matrix of each other workload with every thread; about 10-30 s of CPU work."""
    import ctypes
    import oracle
    orc = oracle.get()
    threads = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
    except OSError:
        gomp = None

    def set_threads(n):
        if gomp is not None:
            gomp.omp_set_num_threads(n)

    d_out, d_in = w_host.shape

    def step_rate(n_rows):
        """Seconds for calibration (rows 0-1023) + encode and decode of n_rows, and the whole-matrix
        rate from them (Mweights/s of encode + decode; extrapolated when n_rows < d_out)."""
        t0 = time.perf_counter()
        sb = orc.sign_mask(sign, d_in)
        sig, _ = orc.calibrate(w_host[:1024], s_host, sb, block)
        t1 = time.perf_counter()
        e = orc.encode(w_host[:n_rows], s_host, sb, block, cb_h, bits, sig, want_idx=False)
        orc.decode(e["codes"], e["norm"], d_in, sig, cb_h, bits, s_host, sb, block)
        t2 = time.perf_counter()
        full = (t1 - t0) + (t2 - t1) * d_out / n_rows
        return t2 - t0, d_out * d_in / full / 1e6

    set_threads(threads)
    runs = [step_rate(d_out) for _ in range(3)]   # the whole step, three times
    t_all = sum(r[0] for r in runs)
    rate_all = float(np.median([r[1] for r in runs]))
    set_threads(1)
    t_one, rate_one = step_rate(1024)
    set_threads(threads)
    others = {}
    for cidx, n_rows in ((0, None), (2, None), (3, None)):
        c = synth.config(cidx)
        mm = c.matrices[0]
        n_rows = mm.d_out if n_rows is None else n_rows
        w = mm.weights(0, n_rows)
        s = mm.channel_scale()
        sb = orc.sign_mask(sign, mm.d_in)
        K = 1 << c.bits[0]
        cb = np.random.default_rng(cidx).standard_normal((K, 2)).astype(np.float32)
        b = c.block
        t0 = time.perf_counter()
        sig = np.full((mm.d_in // 2,), c.fixed_sigma, dtype=np.float32) if c.fixed_sigma else \
            orc.calibrate(w[:1024], s, sb, b)[0]
        e = orc.encode(w, s, sb, b, cb, c.bits[0], sig, want_idx=False)
        orc.decode(e["codes"], e["norm"], mm.d_in, sig, cb, c.bits[0], s, sb, b)
        dt = time.perf_counter() - t0
        others[c.name] = {"Mweights_per_s": round(n_rows * mm.d_in / dt / 1e6, 4), "rows": n_rows, "s": round(dt, 2),
                          "matrix": "%s %dx%d" % (mm.name, mm.d_out, mm.d_in),
                          "note": "sigma given" if c.fixed_sigma else "calibration over rows 0-1023, whole matrix"}
    return {"value": round(rate_all, 3), "unit": "Mweights/s", "cores": threads, "kind": "oracle",
            "sample": "the whole 4096x4096 step (calibration over rows 0-1023, encode and decode of all rows), "
                      "median of 3 runs (%.1f s in all)" % t_all,
            "cpu_model": model, "one_thread": {"value": round(rate_one, 4), "sample": "calibration over rows 0-1023, "
                                               "encode + decode of 1024 rows, whole matrix extrapolated (%.1f s)" % t_one},
            "other_workloads": others}


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

        # one checked call per buffer set, launched directly in the loop (the per-call argument checks
        # of q.qgemm take longer on the host than the product takes on the GPU at these sizes)
        plans = [q.QgemmPlan(x, b["codes"], b["norm"], b["sigma"], cb, bits, scale=scale, sign_seed=sign, block=block,
                             out=y, workspace=ws) for b in sets]

        def fused(i):
            plans[i % n_sets]()

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
        del plans
        res["M%d" % M] = {"qgemm_us": round(t_f * 1e3, 2), "bf16_matmul_us": round(t_b * 1e3, 2),
                          "decode_then_matmul_us": round(t_d * 1e3, 2),
                          "speedup_vs_bf16": round(t_b / t_f, 3), "speedup_vs_decode_matmul": round(t_d / t_f, 3),
                          "hbm_GBps": round(alg / (t_f * 1e-3) / 1e9, 1),
                          "hbm_frac": round(alg / (t_f * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "kernel": "matrix cores (bf16 pieces)"}
        del ws, tmp
    return res


def qgemm13b_run(torch, q, synth, cb, index, bits, block, timed, rot_gib):
    """The fused product on the seven matrices of a 13B-shaped layer (q, k, v, o 5120x5120, gate and up
    13824x5120, down 5120x13824) at M = 1, 4 and 16 activation rows, against hipBLASLt on the decoded
    BF16 matrices; codes and weights rotate over >= rot_gib of copies."""
    dev = cb.device
    c3 = synth.config(3)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    res = {}
    for mm in c3.matrices:
        w = mm.weights_device(dev)
        s = torch.from_numpy(mm.channel_scale()).to(dev)
        e = q.encode(w, cb, bits, index, scale=s, block=block)
        d_out, d_in = w.shape
        per = w.numel() * 2 + e["codes"].numel()
        n = max(2, int(math.ceil(rot_gib * (1 << 30) / per)))
        sets = [{"codes": e["codes"].clone(), "norm": e["norm"], "sigma": e["sigma"],
                 "wd": q.decode(e["codes"], e["norm"], e["sigma"], cb, bits, d_in, scale=s, block=block)} for _ in range(n)]
        del w
        row = {}
        for M in (1, 4, 16):
            x = torch.randn((M, d_in), device=dev, generator=g).to(torch.bfloat16)
            y = torch.empty((M, d_out), dtype=torch.float32, device=dev)
            ws = torch.empty((q.qgemm_workspace(M, d_out, d_in),), dtype=torch.uint8, device=dev)
            plans = [q.QgemmPlan(x, b["codes"], b["norm"], b["sigma"], cb, bits, scale=s, block=block, out=y,
                                 workspace=ws) for b in sets]
            t_f = timed(lambda i: plans[i % n]())
            t_b = timed(lambda i: torch.matmul(x, sets[i % n]["wd"].t()))
            alg = d_out * q.row_stride(d_in, bits) + d_out * 2 + M * d_in * 2 + M * d_out * 4
            row["M%d" % M] = {"qgemm_us": round(t_f * 1e3, 2), "bf16_matmul_us": round(t_b * 1e3, 2),
                              "speedup_vs_bf16": round(t_b / t_f, 3),
                              "hbm_frac": round(alg / (t_f * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
            del plans, ws
        res["%s %dx%d" % (mm.name, d_out, d_in)] = row
        del sets, e
        torch.cuda.empty_cache()
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



if __name__ == "__main__":
    main()
