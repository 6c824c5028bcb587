"""A CPU model of the bonus draw's fp32 rounding, for the flip analysis.

Not a test (pytest does not collect it) and independent of the oracle: it
rebuilds, in numpy, the steps by which the HIP path forms the residual CDF of
one rejected position ("Kangaroo: Self-Speculative Decoding via Shallow
Sub-Networks", "3. Lossless Speculative Verification": the bonus token is
drawn from the normalised max(p - q, 0)), with each fp32 rounding of the GPU
path in place:

  c = fp32(log2 e / T);  o = fp32(max z * c);  exponentials exp2(fp32(z c - o))
  rounded to fp32 and summed in fp64 (the normalisers S_t and D);
  k2 = o_t - o_d + log2(S_t / D) split into fp32 hi + lo;
  d = fp32(fp32(delta c + k_hi) + k_lo);  1 - 2^d by the degree-5 polynomial on
  [-1, 0) or 1 - exp2(d) below;  r = fp32(p_t S_t (1 - 2^d)),

and compares the resulting CDF with the exact one (long double) by drawing
uniforms: the fraction of draws whose token differs is the flip rate per
draw.  Each variant makes one or more of the steps exact, to attribute the
rate.  The model's exp2 is correctly rounded; the GPU's v_exp_f32 is within
about 1 ulp, so the model is a little more accurate than the GPU.  beta = 1.

    python tests/flip_model.py C2 30 2      # workload, sequences, positions
"""
from __future__ import annotations

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from workload.gen import WORKLOADS, make_inputs  # noqa: E402

LOG2E = 1.4426950408889634
# (2^d - 1)/d on [-1, 0), the HIP path's polynomial (fp32 coefficients)
P5 = [6.931471825e-01, 2.402260602e-01, 5.549895018e-02, 9.596269578e-03, 1.290776301e-03,
      1.145800052e-04]
# a cheaper degree-4 fit on [-0.75, 0), measured and rejected
P4 = [6.931471229e-01, 2.402223200e-01, 5.545998737e-02, 9.452956729e-03, 1.074523083e-03]


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def horner(d, coef):
    c = [float(np.float32(v)) for v in coef]
    p = f32(d * c[-1] + c[-2])
    for k in range(len(c) - 3, -1, -1):
        p = f32(d * p + c[k])
    return f32(-d * p)


def exact_cdf(zt, zd, T):
    lt = zt.astype(np.longdouble) / T
    ld = zd.astype(np.longdouble) / T
    p = np.exp(lt - lt.max())
    p /= p.sum()
    q = np.exp(ld - ld.max())
    q /= q.sum()
    r = np.maximum(p - q, 0)
    return np.asarray(np.cumsum(r) / r.sum(), dtype=np.float64)


def model_cdf(zt, zd, T, poly="p5", norm_exact=False, pt_exact=False, c_exact=False, d_exact=False):
    c = LOG2E / T if c_exact else float(np.float32(LOG2E / T))

    def ex(a):
        return f32(2.0 ** a)

    def arg(z, o):
        return f32(z * c - o)

    ot = float(np.float32(zt.max() * c))
    od = float(np.float32(zd.max() * c))
    if norm_exact:
        st = np.exp2(zt.astype(np.longdouble) * c - ot).sum()
        dd = np.exp2(zd.astype(np.longdouble) * c - od).sum()
        k2 = float(ot - od + np.log2(st / dd))
    else:
        k2 = ot - od + np.log2(ex(arg(zt, ot)).sum() / ex(arg(zd, od)).sum())
    khi = float(np.float32(k2))
    klo = float(np.float32(k2 - khi))
    pt = 2.0 ** (zt * c - ot) if pt_exact else ex(arg(zt, ot))
    if d_exact:
        d = (zd - zt) * c + k2
    else:
        d = f32(f32(f32(zd - zt) * c + khi) + klo)
    if poly == "p5":
        omx = np.where(d >= -1, horner(d, P5), f32(1 - ex(d)))
    elif poly == "p4":
        omx = np.where(d >= -0.75, horner(d, P4), f32(1 - ex(d)))
    else:
        omx = -np.expm1(d * np.log(2))
    r = pt * np.clip(omx, 0, 1)
    if not (pt_exact and poly == "exact"):
        r = f32(r)
    return np.cumsum(r) / r.sum()


VARIANTS = {
    "as built": {},
    "degree-4 polynomial": dict(poly="p4"),
    "1 - 2^d exact": dict(poly="exact"),
    "normalisers exact": dict(norm_exact=True),
    "p_t exact": dict(pt_exact=True),
    "c exact": dict(c_exact=True),
    "all exact but c": dict(norm_exact=True, pt_exact=True, poly="exact", d_exact=True),
    "all exact": dict(norm_exact=True, pt_exact=True, poly="exact", d_exact=True, c_exact=True),
}


def main(name: str, nseq: int, npos: int, draws: int = 100_000) -> None:
    w = WORKLOADS[name].sized(B=nseq, beta=1.0)
    inp = make_inputs(w, seed=11)
    T = inp["temperature"].double().numpy()
    tg = inp["target"].float().numpy().astype(np.float64)
    dr = inp["draft"].float().numpy().astype(np.float64)
    rng = np.random.default_rng(0)
    flips = {k: 0 for k in VARIANTS}
    n = 0
    for b in range(nseq):
        if w.identical_every and b % w.identical_every == 0:
            continue
        Tb = float(np.float32(T[b]))
        for pos in range(min(npos, w.K)):
            ce = exact_cdf(tg[b, pos], dr[b, pos], Tb)
            u = rng.random(draws)
            want = np.searchsorted(ce, u)
            n += u.size
            for k, kw in VARIANTS.items():
                got = np.searchsorted(model_cdf(tg[b, pos], dr[b, pos], Tb, **kw), u)
                flips[k] += int((got != want).sum())
    for k in VARIANTS:
        print(f"{name} {k:22s} flips per draw {flips[k] / n:.2e} ({flips[k]} of {n})")


if __name__ == "__main__":
    main(sys.argv[1], int(sys.argv[2]) if len(sys.argv) > 2 else 20,
         int(sys.argv[3]) if len(sys.argv) > 3 else 2)
