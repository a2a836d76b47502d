"""GPU parity of the activation-aware channel scale (reading R11) against the CPU oracle.

r_j within 1e-14 relative (fp64 sums in another order); s_j = fl32(r_j^alpha) within one fp32 ulp
(pow in fp64 differs by a few ulps between the device library and the host's, which can move the
fp32 rounding); s_j = 1 exactly for a dead channel.  Cases: one row, ragged row counts, widths that
are not multiples of the 4-column lanes, fp32 and BF16, padded leading dimensions, several alpha.
End to end: the scale from the GPU lowers the codec's layer-output error (the trace-identity
quantity ||X dW^T||^2) against s = 1 on activations with strong channels.
"""
import numpy as np
import pytest
import torch

from helpers import DEV, log, t

pytestmark = pytest.mark.gpu


def _acts(seed, T, d_in):
    rng = np.random.default_rng(seed)
    rho = np.exp(0.5 * rng.standard_normal(d_in))
    rho[rng.choice(d_in, max(1, d_in // 100), replace=False)] *= 30
    x = (rng.standard_normal((T, d_in)) * rho).astype(np.float32)
    if d_in > 3:
        x[:, 3] = 0   # a dead channel
    return x


@pytest.mark.parametrize("T,d_in,dtype,alpha,ld", [
    (1, 64, "fp32", 0.3, None), (17, 7, "bf16", 0.3, None), (2048, 4096, "bf16", 0.3, None),
    (300, 5000, "fp32", 0.5, None), (129, 1000, "bf16", 1.0, 1000 + 12), (64, 4096, "fp32", -0.5, 4096 + 4),
    (5000, 256, "bf16", 0.0, None)])
def test_act_scale_matches_oracle(q, orc, T, d_in, dtype, alpha, ld):
    x = _acts(T + d_in, T, d_in)
    if dtype == "bf16":
        xt = torch.from_numpy(x).to(torch.bfloat16)
        x = xt.float().numpy()
    else:
        xt = torch.from_numpy(x)
    if ld is not None:
        big = torch.zeros((T, ld), dtype=xt.dtype)
        big[:, :d_in] = xt
        xd = big.to(DEV)[:, :d_in]
    else:
        xd = xt.to(DEV)
    log("act scale T=%d d_in=%d %s alpha=%g ld=%s" % (T, d_in, dtype, alpha, ld))
    s, r = q.act_scale(xd, alpha, want_rms=True)
    torch.cuda.synchronize()
    s, r = s.cpu().numpy(), r.cpu().numpy()
    s_ref, r_ref = orc.act_scale(x, alpha)
    np.testing.assert_allclose(r, r_ref, rtol=1e-14, atol=0)
    ulp = np.abs(s.view(np.int32).astype(np.int64) - s_ref.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1, ulp.max()
    if d_in > 3:
        assert s[3] == 1.0 and r[3] == 0.0
    log("  %d of %d scales differ by one ulp" % (int((ulp != 0).sum()), d_in))


def test_act_scale_lowers_the_output_error(q, orc):
    rng = np.random.default_rng(21)
    T, d_out, d_in, block, bits = 512, 256, 1024, 128, 8
    x = _acts(5, T, d_in)
    w = (rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32)
    seed = 977   # sign-mask seed
    cb, _ = q.codebook_train(t(rng.standard_normal((1 << 16, 2)).astype(np.float32)), bits, 30)
    idx = q.codebook_index(cb, bits)
    xd, wd = t(x), t(w)
    err = {}
    for name, s in (("plain", torch.ones(d_in, device=DEV)), ("aware", q.act_scale(xd, 0.3))):
        e = q.encode(wd, cb, bits, idx, scale=s, sign_seed=seed, block=block)
        wh = q.decode(e["codes"], e["norm"], e["sigma"], cb, bits, d_in, scale=s, sign_seed=seed,
                      block=block, out_dtype=torch.float32)
        err[name] = float(torch.sum((xd @ (wh - wd).t()) ** 2))
    log("  output error: s = 1 %.4g, s = r^0.3 %.4g" % (err["plain"], err["aware"]))
    assert err["aware"] < 0.8 * err["plain"]
