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
    """oracle Factor -> device Factor (fp32 values; what the device sees)."""
    coef = np.zeros(fg.COEF_COUNT, dtype=np.float32)
    coef[fg.COEF_ALPHA] = f.alpha
    coef[fg.COEF_BETA] = f.beta
    coef[fg.COEF_LAMBDA_ISO] = f.lambda_iso
    coef[fg.COEF_LAMBDA_FLOOR] = f.lambda_floor
    coef[fg.COEF_TRACE] = f.trace
    coef[fg.COEF_SIGMA2_TAIL] = f.sigma2_tail
    coef[fg.COEF_DW:fg.COEF_DW + fg.RANK] = f.d_w
    coef[fg.COEF_DU:fg.COEF_DU + fg.RANK] = f.d_u
    df = fg.Factor(f.d_in, U=torch.from_numpy(np.ascontiguousarray(f.U, dtype=np.float32)).to(DEV),
                   theta=torch.from_numpy(np.asarray(f.theta, dtype=np.float32)).to(DEV),
                   coef=torch.from_numpy(coef).to(DEV))
    if df.packs is not None:
        fg.gift_prepare_factor(df)
    return df


def factor_host(df):
    """device Factor -> (U, alpha, beta, D_w, D_u) as the fp32 values it holds."""
    U = df.U.cpu().numpy()
    c = df.coef.cpu().numpy()
    return (U, float(c[fg.COEF_ALPHA]), float(c[fg.COEF_BETA]),
            c[fg.COEF_DW:fg.COEF_DW + fg.RANK].copy(), c[fg.COEF_DU:fg.COEF_DU + fg.RANK].copy())


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(msg):
    print("[gpu-case] " + msg, flush=True)
