"""Helpers for the device tests: move seeded inputs to the GPU, build layers,
read results back for the oracle."""

import numpy as np
import torch

import fac_whitening_gift_amd as fg

DEV = "cuda"


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def upload_factor(f):
    """oracle Factor -> device Factor (fp32 values; what the device sees).
    An oracle factor of r <= 32 columns fills a 32-column factor, of up to 64
    a 64-column one (zero columns after r)."""
    r = f.U.shape[1]
    cols = fg.factor_cols(r)
    coef = np.zeros(8 + 2 * cols, dtype=np.float32)
    coef[fg.COEF_ALPHA] = f.alpha
    coef[fg.COEF_BETA] = f.beta
    coef[fg.COEF_LAMBDA_ISO] = f.lambda_iso
    coef[fg.COEF_LAMBDA_FLOOR] = f.lambda_floor
    coef[fg.COEF_TRACE] = f.trace
    coef[fg.COEF_SIGMA2_TAIL] = f.sigma2_tail
    coef[fg.COEF_DW:fg.COEF_DW + r] = f.d_w
    coef[fg.COEF_DW + cols:fg.COEF_DW + cols + r] = f.d_u
    U = np.zeros((f.d_in, cols), dtype=np.float32)
    U[:, :r] = f.U
    th = np.zeros(cols, dtype=np.float32)
    th[:r] = f.theta
    df = fg.Factor(f.d_in, U=torch.from_numpy(U).to(DEV), theta=torch.from_numpy(th).to(DEV),
                   coef=torch.from_numpy(coef).to(DEV), rank=max(r, 1))
    if df.packs is not None:
        fg.gift_prepare_factor(df)
    return df


def factor_host(df):
    """device Factor -> (U, alpha, beta, D_w, D_u) as the fp32 values it holds."""
    U = df.U.cpu().numpy()
    c = df.coef.cpu().numpy()
    k = df.cols
    return (U, float(c[fg.COEF_ALPHA]), float(c[fg.COEF_BETA]),
            c[fg.COEF_DW:fg.COEF_DW + k].copy(), c[fg.COEF_DW + k:fg.COEF_DW + 2 * k].copy())


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(msg):
    print("[gpu-case] " + msg, flush=True)
