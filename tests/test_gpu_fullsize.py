"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

Every case encodes (with calibration) and decodes a whole matrix on the GPU, exactly as the
benchmark step does. The oracle is too slow to redo a whole matrix, so it checks:
  * sigma over every pair (the oracle calibrates on the same first min(d_out, 1024) rows);
  * codes and norms of a seeded sample of rows, which always includes the first and last rows;
  * the BF16 decode of the sampled rows, decoding the GPU's codes on both sides;
  * the fp32 decode of a few rows.
The comparison rules are those of tests/helpers.py.

Matrices and codebooks:
  * the 4096x4096 attention projection, and the 11008x4096 / 4096x11008 MLP pair with its
    retrained codebook (2^22 points, 50 iterations, b = 256);
  * the seven matrices of a 13B layer at B = 11 (the K = 2048 codebook of the 4096x4096 workload)
    and two of them at B = 7 (K = 128);
  * two matrices from the 40-layer stack (its first and last layer);
  * the 256x512 fp32 matrix with sigma fixed at 1/8, compared over all rows.
"""
import os

import numpy as np
import pytest
import torch

from helpers import DEV, assert_bf16_within_1ulp, assert_rel_l2, check_indices, log, sign_tensor, t, unpack_rows

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# id: (config index, matrix selector, bits, golden codebook, sampled rows)
CASES = {
    "attn4096_b11": (1, 0, 11, "cb_cfg1_k2048", 48),
    "mlp_up_11008x4096_b11": (2, 0, 11, "cb_cfg2_k2048", 40),
    "mlp_down_4096x11008_b11": (2, 1, 11, "cb_cfg2_k2048", 40),
    "l13b_q_5120x5120_b11": (3, 0, 11, "cb_cfg1_k2048", 32),
    "l13b_k_5120x5120_b11": (3, 1, 11, "cb_cfg1_k2048", 24),
    "l13b_v_5120x5120_b11": (3, 2, 11, "cb_cfg1_k2048", 24),
    "l13b_o_5120x5120_b11": (3, 3, 11, "cb_cfg1_k2048", 24),
    "l13b_gate_13824x5120_b11": (3, 4, 11, "cb_cfg1_k2048", 24),
    "l13b_up_13824x5120_b11": (3, 5, 11, "cb_cfg1_k2048", 24),
    "l13b_down_5120x13824_b11": (3, 6, 11, "cb_cfg1_k2048", 24),
    "l13b_q_5120x5120_b7": (3, 0, 7, "cb_cfg3_k128", 24),
    "l13b_down_5120x13824_b7": (3, 6, 7, "cb_cfg3_k128", 24),
    "stack40_L0_gate_b11": (4, (0, 4), 11, "cb_cfg1_k2048", 16),
    "stack40_L39_down_b11": (4, (39, 6), 11, "cb_cfg1_k2048", 16),
    "small256x512_fp32_b8": (0, 0, 8, "cb_cfg0_k256", None),
}


def _codebook(name):
    d = np.load(os.path.join(GOLDEN, name + ".npz"))
    return np.ascontiguousarray(d["codebook"]).astype(np.float32)


def _matrix(synth, cfg_i, sel):
    if cfg_i == 4:
        layer, m = sel
        return synth.config(4, n_layers=layer + 1).matrices[7 * layer + m], synth.config(4).block
    cfg = synth.config(cfg_i)
    return cfg.matrices[sel], cfg.block


def _sample_rows(d_out, n, seed):
    if n is None or n >= d_out:
        return np.arange(d_out)
    rng = np.random.default_rng(seed)
    edge = list(range(4)) + list(range(d_out - 4, d_out))
    mid = rng.choice(np.arange(4, d_out - 4), size=n - len(edge), replace=False)
    return np.unique(np.concatenate([edge, mid])).astype(np.int64)


def _ulp_f32(a, b):
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


@pytest.mark.parametrize("case", list(CASES), ids=list(CASES))
def test_fullsize_parity(q, orc, synth, case):
    cfg_i, sel, bits, cb_name, n_rows = CASES[case]
    spec, block = _matrix(synth, cfg_i, sel)
    d_out, d_in = spec.d_out, spec.d_in
    log("fullsize %s: %dx%d bits=%d block=%d" % (case, d_out, d_in, bits, block))
    cb = _codebook(cb_name)
    w = spec.weights()
    s = spec.channel_scale()
    sb = synth.sign_bits(d_in)
    fixed_sigma = synth.config(cfg_i).fixed_sigma if cfg_i != 4 else None

    # ---- GPU: the benchmark's calls on the whole matrix
    if spec.bf16:
        w_dev = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        w_dev = t(w)
    cb_dev = t(cb)
    index = q.codebook_index(cb_dev, bits)
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    sig_in = None if fixed_sigma is None else t(np.full(d_in // 2, fixed_sigma, np.float32))
    enc = q.encode(w_dev, cb_dev, bits, index, scale=t(s), sign_bits=sign_tensor(sb), block=block,
                   sigma=sig_in, status=st)
    dec = q.decode(enc["codes"], enc["norm"], enc["sigma"], cb_dev, bits, d_in, scale=t(s),
                   sign_bits=sign_tensor(sb), block=block)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    sigma = enc["sigma"].cpu().numpy()
    rows = _sample_rows(d_out, n_rows, 1000 + cfg_i)
    ridx = torch.from_numpy(rows).to(DEV)
    codes = enc["codes"].index_select(0, ridx).cpu().numpy()
    norm = enc["norm"].index_select(0, ridx).cpu().numpy().view(np.uint16)
    dec16 = dec.index_select(0, ridx).view(torch.int16).cpu().numpy().view(np.uint16)
    assert not torch.isnan(dec.float()).any().item()
    del dec, w_dev

    # ---- sigma over every pair
    if fixed_sigma is None:
        sig_ref, st_ref = orc.calibrate(w[: min(d_out, 1024)], s, sb, block)
        assert st_ref == 0
        ulp = _ulp_f32(sigma, sig_ref)
        assert ulp.max() <= 1, "sigma differs by %d ulp" % ulp.max()
        log("  sigma: %d of %d pairs differ by 1 ulp" % (int((ulp != 0).sum()), sigma.size))

    # ---- codes and norms of the sampled rows (the oracle encodes with the GPU's sigma)
    ws = w[rows]
    ref = orc.encode(ws, s, sb, block, cb, bits, sigma, want_p=True)
    np.testing.assert_array_equal(norm, ref["norm"])
    gidx = unpack_rows(orc, codes, bits, d_in)
    flips = check_indices(gidx, ref["idx"], ref["p"], cb)
    log("  codes: %d rows, %d near-tie index flips" % (rows.size, flips))

    # ---- decode of the sampled rows: both sides decode the GPU's codes
    dref = orc.decode(codes, norm, d_in, sigma, cb, bits, s, sb, block)
    n_diff = assert_bf16_within_1ulp(dec16, dref["bf16"])
    log("  decode: %d of %d BF16 outputs differ by 1 ulp" % (n_diff, dec16.size))
    few = min(4, rows.size)
    got32 = q.decode(t(codes[:few]), t(norm[:few].view(np.int16)), t(sigma), cb_dev, bits, d_in, scale=t(s),
                     sign_bits=sign_tensor(sb), block=block, out_dtype=torch.float32).cpu().numpy()
    assert_rel_l2(got32, dref["f32"][:few], 1e-5)
