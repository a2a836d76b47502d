"""Shared helpers of the GPU parity tests: marshalling numpy inputs through the C ABI binding,
and the comparison rules against the CPU oracle.

Comparison rules (tolerances of the codec's parity contract):
  * indices: equal, except at near-ties -- a different index is accepted only when its fp32
    distance to the oracle's pair exceeds the oracle's by at most 1e-6 relative;
  * sigma and f16 row norms: within one unit in the last place (expected equal);
  * fp32 reconstruction: relative L2 error at most 1e-5;
  * BF16 reconstruction: every element within one BF16 ulp.
"""
import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def t(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def w_tensor(w: np.ndarray, ld: int = None) -> torch.Tensor:
    """float32 array or uint16 bf16 bit patterns -> device tensor (optionally with row padding)."""
    if w.dtype == np.uint16:
        x = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).view(torch.bfloat16)
    else:
        x = torch.from_numpy(np.ascontiguousarray(w))
    if ld is not None and ld != w.shape[1]:
        big = torch.full((w.shape[0], ld), float("nan"), dtype=x.dtype)
        big[:, : w.shape[1]] = x
        return big.to(DEV)[:, : w.shape[1]]
    return x.to(DEV)


def gpu_encode(q, w, s, seed, block, cb, bits, sigma=None, ld=None, index=None, cb_dev=None):
    """GPU encode through the binding; `seed` is the sign-mask seed (None: the library default)."""
    cb_dev = t(cb) if cb_dev is None else cb_dev
    index = q.codebook_index(cb_dev, bits) if index is None else index
    st = torch.zeros((1,), dtype=torch.int32, device=DEV)
    out = q.encode(w_tensor(w, ld), cb_dev, bits, index, scale=None if s is None else t(s),
                   sign_seed=q.DEFAULT_SIGN_SEED if seed is None else seed, block=block,
                   sigma=None if sigma is None else t(sigma), status=st)
    torch.cuda.synchronize()
    return {"codes": out["codes"].cpu().numpy(), "norm": out["norm"].cpu().numpy().view(np.uint16),
            "sigma": out["sigma"].cpu().numpy(), "status": int(st.item())}


def gpu_decode(q, codes, norm, sigma, cb, bits, s, seed, d_in, block, out_dtype=torch.bfloat16, ld=None):
    d_out = norm.shape[0]
    out = None
    if ld is not None and ld != d_in:
        out = torch.full((d_out, ld), 7.0, dtype=out_dtype, device=DEV)[:, :d_in]
    res = q.decode(t(codes), t(norm.view(np.int16)), t(sigma), t(cb), bits, d_in, scale=None if s is None else t(s),
                   sign_seed=q.DEFAULT_SIGN_SEED if seed is None else seed, block=block, out_dtype=out_dtype,
                   out=out)
    torch.cuda.synchronize()
    if out_dtype == torch.bfloat16:
        return res.view(torch.int16).cpu().numpy().view(np.uint16)
    return res.cpu().numpy()


def unpack_rows(orc, codes, bits, d_in):
    return np.stack([orc.unpack_row(codes[i], bits, d_in) for i in range(codes.shape[0])])


def fp32_dist(p, c):
    """Squared distance with the codec's fp32 rounding: fl(fl(dx*dx) + fl(dy*dy))."""
    p = p.astype(np.float32)
    c = c.astype(np.float32)
    dx = (p[..., 0] - c[..., 0]).astype(np.float32)
    dy = (p[..., 1] - c[..., 1]).astype(np.float32)
    return (dx * dx).astype(np.float32) + (dy * dy).astype(np.float32)


def check_indices(gpu_idx, ref_idx, p_ref, cb, rows=None):
    """Indices equal except at near-ties (relative distance gap <= 1e-6).  Returns #tie flips."""
    gpu_idx = np.asarray(gpu_idx)
    ref_idx = np.asarray(ref_idx)
    mism = gpu_idx != ref_idx
    n = int(mism.sum())
    if n:
        p = p_ref.reshape(gpu_idx.shape + (2,))[mism]
        dg = fp32_dist(p, cb[gpu_idx[mism]]).astype(np.float64)
        dr = fp32_dist(p, cb[ref_idx[mism]]).astype(np.float64)
        bad = dg - dr > 1e-6 * dr
        assert not bad.any(), "index mismatch beyond the near-tie bound at %d of %d pairs: gpu %s ref %s" % (
            int(bad.sum()), gpu_idx.size, gpu_idx[mism][bad][:5], ref_idx[mism][bad][:5])
    return n


def bf16_ordinal(u16):
    u = u16.astype(np.int32)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)


def assert_bf16_within_1ulp(got, ref):
    d = np.abs(bf16_ordinal(got) - bf16_ordinal(ref))
    assert d.max() <= 1, "BF16 differs by %d ulp at %s" % (d.max(), np.argwhere(d == d.max())[:3])
    return int((d != 0).sum())


def assert_rel_l2(got, ref, tol=1e-5):
    num = np.linalg.norm((got.astype(np.float64) - ref.astype(np.float64)).ravel())
    den = np.linalg.norm(ref.astype(np.float64).ravel())
    rel = num / den if den > 0 else num
    assert rel <= tol, "relative L2 error %.3g > %.1g" % (rel, tol)
    return rel
