"""GIFT round trip, step by step, in fp64 numpy (oracle; test infrastructure only).

What the method computes (GIFT review, "What carries the argument" and
"Core claim"): each selected layer's weight gradient G (d_out x d_in) is
moved into a near-isotropic coordinate system with the input-side K-FAC
factor A = E[a a^T] before FP8 quantization, and mapped back afterwards; the
factor is approximated at rank 32 (free-parameter ledger) and refreshed
every 50 steps (ledger; referee report major comment 2 on Algorithm 1).
The baseline quantizes G directly with a single per-tensor FP8 scale
("The pith": one scale must stretch over the largest direction).

The pages print no formula, so the concrete steps below are this
implementation's reading, each marked where it is taken:

1. A = X^T X / N from the layer inputs X (N x d_in).
2. t = tr(A); lambda_floor = eps * t / d_in (eps = 1e-3).
3. Top-r eigenpairs of A by randomized subspace iteration from a Gaussian
   sketch Omega (d_in x l, l = 64): Q = orth(A Omega), then `power_steps`
   times Q = orth(A Q), then Rayleigh-Ritz on B = Q^T A Q.  Theta = the r
   largest Ritz values clamped at 0, U = Q V[:, :r].
4. Damping: A_r = U diag(Theta) U^T + lambda_iso I.  Reading "floor+tail"
   (default): lambda_iso = lambda_floor + mean of the discarded spectrum,
   (t - sum Theta) / (d_in - r), the isotropic residual of probabilistic
   PCA; reading "floor": lambda_iso = lambda_floor.  lambda_iso is kept at
   or above 1e-30 so an all-zero input (t = 0) still gives finite
   coefficients (whitening then reduces to a scalar multiple).
5. Whitening is input-side, G -> G A_r^{-1/2}; un-whitening is
   W -> W A_r^{1/2}.  With U orthonormal,
   A_r^{-1/2} = alpha I + U diag(D_w) U^T, alpha = lambda_iso^{-1/2},
   D_w = (Theta + lambda_iso)^{-1/2} - lambda_iso^{-1/2};
   A_r^{1/2}  = beta I + U diag(D_u) U^T,  beta = lambda_iso^{1/2},
   D_u = (Theta + lambda_iso)^{1/2} - lambda_iso^{1/2}.
6. Per-tensor E4M3 quantization of the whitened fp32 tensor W:
   amax = max |W|; scale = fl32(448 / amax); inv = fl32(amax / 448);
   code = E4M3(fl32(W * scale)); amax == 0 gives scale = inv = 1.  A
   finite amax so small that 448 / amax overflows fp32 (below 448 /
   FLT_MAX, about 1.3e-36) gets the largest finite fp32 as its scale, so
   zeros stay zeros and no finite input turns into a NaN code (reading).
7. Dequantize W^ = fl32(decode(code) * inv); un-whiten G^ = W^ A_r^{1/2}.
8. A data-parallel reduction of R payloads (the ranks' quantized whitened
   gradients summed in the collective) is read as fp32 additions of the
   dequantized payloads in rank order, then one un-whitening of the sum.
9. The FP4 payload (the direction the review expects larger gains in) is
   the same round trip with the whitened tensor stored as OCP MXFP4
   (oracle/mxfp4.py: E2M1 elements, one power-of-two scale per 32
   elements of a row).
10. Block-diagonal factor "block-A-b" (the review's round-trip error table
   names block-A-32 and block-A-64 without defining them; reading): A is
   replaced by its d_in/b diagonal b x b blocks A_i, each damped by
   lambda_floor and used in full: W[:, block i] = G[:, block i] S_i with
   S_i = (A_i + lambda_floor I)^{-1/2}, and G^[:, block i] =
   W^[:, block i] (A_i + lambda_floor I)^{1/2}.  A block keeps its whole
   spectrum, so there is no discarded tail to add to the damping.
11. Full-rank and two-sided references (the review's claim that the
   input-side factor captures nearly all of the full two-sided K-FAC
   transform's benefit, "The pith", and its Eq. 14 Cholesky form L_A^-T):
   input-side symmetric W = G (A + lambda I)^{-1/2}; input-side Cholesky
   W = G L^-T with L L^T = A + lambda I, undone by W^ L^T; two-sided
   W = (B + mu I)^{-1/2} G (A + lambda I)^{-1/2} with the output-side factor
   read as the gradient's row second moment B = G G^T / d_in and
   mu = eps tr(B) / d_out (reading: the pages give no output-side
   generator).  Each is quantized like W of step 6.

Precision: inputs are fp32 (activations bf16 values held in fp32); every
linear-algebra step runs in fp64.  The steps that decide an integer (the
amax, the scale and the E4M3 code) run in fp32, the precision the device
takes them in.
"""

from dataclasses import dataclass, field

import numpy as np

from . import e4m3
from . import mxfp4

RANK = 32
SKETCH_WIDTH = 64
POWER_STEPS = 4
DAMP_EPS = 1e-3
BLOCK = 128
LAMBDA_MIN = 1e-30

DAMPING_FLOOR = "floor"
DAMPING_FLOOR_PLUS_TAIL = "floor+tail"

FLAG_NONFINITE = 1
FLAG_ZERO_AMAX = 2


# --------------------------------------------------------------------------
# factor refresh
# --------------------------------------------------------------------------

def covariance(X):
    """A = X^T X / N in fp64 (step 1; GIFT review, "What carries the
    argument": the input-side factor is the second moment of layer inputs)."""
    X = np.asarray(X, dtype=np.float64)
    return X.T @ X / X.shape[0]


def trace_floor(A, eps=DAMP_EPS):
    """t = tr(A) and lambda_floor = eps * t / d (step 2)."""
    t = float(np.trace(A))
    return t, eps * t / A.shape[0]


def orth(Y):
    """Orthonormal basis of the columns of Y (Householder QR, reduced)."""
    q, _ = np.linalg.qr(Y)
    return q


def subspace_iteration(A, omega, power_steps=POWER_STEPS):
    """Q = orth(A Omega), then power_steps times Q = orth(A Q) (step 3)."""
    Q = orth(A @ omega)
    for _ in range(power_steps):
        Q = orth(A @ Q)
    return Q


def rayleigh_ritz(A, Q, rank=RANK):
    """Ritz pairs of A on span(Q), largest first: (theta[rank], U[d, rank]).

    Theta is clamped at 0 (A is positive semi-definite, so only rounding can
    make a Ritz value negative).
    """
    B = Q.T @ A @ Q
    B = 0.5 * (B + B.T)
    w, V = np.linalg.eigh(B)
    order = np.argsort(w)[::-1][:rank]
    theta = np.maximum(w[order], 0.0)
    U = Q @ V[:, order]
    return theta, U


def damping(t, theta, d, eps=DAMP_EPS, mode=DAMPING_FLOOR_PLUS_TAIL):
    """(lambda_iso, lambda_floor, sigma2_tail) of step 4."""
    r = len(theta)
    lam_floor = eps * t / d
    tail = max(0.0, (t - float(np.sum(theta))) / (d - r)) if d > r else 0.0
    if mode == DAMPING_FLOOR_PLUS_TAIL:
        lam = lam_floor + tail
    elif mode == DAMPING_FLOOR:
        lam = lam_floor
    else:
        raise ValueError(mode)
    return max(lam, LAMBDA_MIN), lam_floor, tail


def coefficients(theta, lam):
    """alpha, beta, D_w, D_u of step 5, written as the plain differences."""
    theta = np.asarray(theta, dtype=np.float64)
    alpha = lam ** -0.5
    beta = lam ** 0.5
    d_w = (theta + lam) ** -0.5 - alpha
    d_u = (theta + lam) ** 0.5 - beta
    return alpha, beta, d_w, d_u


@dataclass
class Factor:
    """Rank-r input-side factor A_r = U diag(theta) U^T + lambda_iso I."""
    U: np.ndarray                 # d_in x r, orthonormal columns
    theta: np.ndarray             # r, descending, >= 0
    lambda_iso: float
    lambda_floor: float
    trace: float
    sigma2_tail: float
    alpha: float = field(init=False)
    beta: float = field(init=False)
    d_w: np.ndarray = field(init=False)
    d_u: np.ndarray = field(init=False)

    def __post_init__(self):
        self.alpha, self.beta, self.d_w, self.d_u = coefficients(
            self.theta, self.lambda_iso)

    @property
    def d_in(self):
        return self.U.shape[0]

    def dense(self):
        """A_r as a dense d x d matrix (fp64)."""
        return (self.U * self.theta) @ self.U.T + self.lambda_iso * np.eye(self.d_in)


def refresh_factor(X, omega, rank=RANK, eps=DAMP_EPS,
                   power_steps=POWER_STEPS, mode=DAMPING_FLOOR_PLUS_TAIL,
                   A=None):
    """Steps 1-5: activations X (N x d_in) and sketch Omega -> Factor."""
    if A is None:
        A = covariance(X)
    t, _ = trace_floor(A, eps)
    Q = subspace_iteration(A, np.asarray(omega, dtype=np.float64), power_steps)
    theta, U = rayleigh_ritz(A, Q, rank)
    lam, lam_floor, tail = damping(t, theta, A.shape[0], eps, mode)
    return Factor(U=U, theta=theta, lambda_iso=lam, lambda_floor=lam_floor,
                  trace=t, sigma2_tail=tail)


def factor_from_parts(U, theta, lambda_iso, lambda_floor=0.0, trace=0.0,
                      sigma2_tail=0.0):
    """Factor from given U, Theta and lambda_iso (e.g. read back from a device)."""
    return Factor(U=np.asarray(U, dtype=np.float64),
                  theta=np.asarray(theta, dtype=np.float64),
                  lambda_iso=float(lambda_iso), lambda_floor=float(lambda_floor),
                  trace=float(trace), sigma2_tail=float(sigma2_tail))


# --------------------------------------------------------------------------
# whitening (step 5)
# --------------------------------------------------------------------------

def whiten_with(G, U, alpha, d_w):
    """W = alpha G + (G U) diag(D_w) U^T  (= G A_r^{-1/2}), fp64."""
    G = np.asarray(G, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    return alpha * G + ((G @ U) * np.asarray(d_w, dtype=np.float64)) @ U.T


def unwhiten_with(W, U, beta, d_u):
    """G = beta W + (W U) diag(D_u) U^T  (= W A_r^{1/2}), fp64."""
    W = np.asarray(W, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    return beta * W + ((W @ U) * np.asarray(d_u, dtype=np.float64)) @ U.T


def whiten(G, f):
    return whiten_with(G, f.U, f.alpha, f.d_w)


def unwhiten(W, f):
    return unwhiten_with(W, f.U, f.beta, f.d_u)


# --------------------------------------------------------------------------
# quantization (step 6-7)
# --------------------------------------------------------------------------

def amax(w32):
    """max |w| of an fp32 array, as fp32.

    Taken as the largest IEEE bit pattern of |w|, which is the ordinary
    maximum for finite tensors and lets NaN dominate +inf dominate finite
    values (the reading for non-finite inputs).
    """
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    if w32.size == 0:
        return np.float32(0.0)
    bits = w32.view(np.uint32) & np.uint32(0x7FFFFFFF)
    return np.array([bits.max()], dtype=np.uint32).view(np.float32)[0]


def scale_from_amax(a):
    """(scale, inv, flags) for one amax (fp32 arithmetic, IEEE division)."""
    a = np.float32(a)
    flags = 0
    if not np.isfinite(a):
        flags |= FLAG_NONFINITE
    if a == 0:
        return np.float32(1.0), np.float32(1.0), flags | FLAG_ZERO_AMAX
    with np.errstate(all="ignore"):
        scale = np.float32(np.float32(e4m3.MAX_FINITE) / a)
        inv = a / np.float32(e4m3.MAX_FINITE)
    if np.isfinite(a) and np.isinf(scale):
        scale = np.finfo(np.float32).max   # 448 / amax overflows: largest finite scale
    return np.float32(scale), np.float32(inv), flags


def quantize_tensor(w32):
    """Per-tensor E4M3: fp32 tensor -> (codes uint8, inv fp32, flags)."""
    w32 = np.asarray(w32, dtype=np.float32)
    scale, inv, flags = scale_from_amax(amax(w32))
    with np.errstate(all="ignore"):
        y = (w32 * scale).astype(np.float32)
    return e4m3.encode(y), inv, flags


def dequantize_tensor(codes, inv):
    """W^ = fl32(decode(code) * inv)."""
    with np.errstate(all="ignore"):
        return (e4m3.decode(codes) * np.float32(inv)).astype(np.float32)


def quantize_block128(w32):
    """1 x 128 block scaling: one scale per 128 consecutive elements of a row.

    Returns (codes d_out x d_in, inv d_out x d_in/128 fp32, flags).  Each
    segment is quantized exactly as a per-tensor quantization of that segment
    alone.
    """
    w32 = np.asarray(w32, dtype=np.float32)
    d_out, d_in = w32.shape
    if d_in % BLOCK:
        raise ValueError("d_in must be a multiple of 128 for block scaling")
    nb = d_in // BLOCK
    codes = np.empty((d_out, d_in), dtype=np.uint8)
    inv = np.empty((d_out, nb), dtype=np.float32)
    flags = 0
    for i in range(d_out):
        for b in range(nb):
            seg = w32[i, b * BLOCK:(b + 1) * BLOCK]
            c, s_inv, f = quantize_tensor(seg)
            codes[i, b * BLOCK:(b + 1) * BLOCK] = c
            inv[i, b] = s_inv
            flags |= f
    return codes, inv, flags


def dequantize_block128(codes, inv):
    """W^ = fl32(decode(code) * inv of the code's 128-element row segment)."""
    codes = np.asarray(codes, dtype=np.uint8)
    inv_full = np.repeat(np.asarray(inv, dtype=np.float32), BLOCK, axis=1)
    with np.errstate(all="ignore"):
        return (e4m3.decode(codes) * inv_full).astype(np.float32)


def quantize(w32, block128=False):
    return quantize_block128(w32) if block128 else quantize_tensor(w32)


def dequantize(codes, inv, block128=False):
    return dequantize_block128(codes, inv) if block128 else dequantize_tensor(codes, inv)


# --------------------------------------------------------------------------
# round trips
# --------------------------------------------------------------------------

def euclid_roundtrip(G, block128=False):
    """Euclidean baseline: quantize G itself -> (codes, inv, G^ fp32, flags)."""
    G32 = np.asarray(G, dtype=np.float32)
    codes, inv, flags = quantize(G32, block128)
    return codes, inv, dequantize(codes, inv, block128), flags


def gift_roundtrip(G, f, block128=False):
    """GIFT: whiten -> fl32 -> quantize -> dequantize -> un-whiten.

    Returns (codes, inv, W32, G^ fp64, flags).
    """
    W32 = whiten(G, f).astype(np.float32)
    codes, inv, flags = quantize(W32, block128)
    What = dequantize(codes, inv, block128)
    return codes, inv, W32, unwhiten(What, f), flags


def euclid_roundtrip_mx(G):
    """Euclidean MXFP4: (codes, scales, G^ fp32, flags)."""
    G32 = np.asarray(G, dtype=np.float32)
    codes, scales, flags = mxfp4.quantize(G32)
    return codes, scales, mxfp4.dequantize(codes, scales), flags


def gift_roundtrip_mx(G, f):
    """GIFT with an MXFP4 payload: whiten -> fl32 -> MXFP4 -> dequantize ->
    un-whiten.  Returns (codes, scales, W32, G^ fp64, flags)."""
    W32 = whiten(G, f).astype(np.float32)
    codes, scales, flags = mxfp4.quantize(W32)
    return codes, scales, W32, unwhiten(mxfp4.dequantize(codes, scales), f), flags


# --------------------------------------------------------------------------
# block-diagonal factor (step 10)
# --------------------------------------------------------------------------

@dataclass
class BlockFactor:
    """S and S^-1 of every diagonal block, stacked: rows b*i .. b*i+b-1 of
    S (d_in x b) hold S_i = (A_i + lambda I)^{-1/2}, likewise S_inv; theta
    holds each block's eigenvalues, descending within the block."""
    S: np.ndarray
    S_inv: np.ndarray
    theta: np.ndarray
    lambda_iso: float
    trace: float

    @property
    def b(self):
        return self.S.shape[1]


def block_factor(A, b, eps=DAMP_EPS):
    """Step 10: per diagonal block, eigh, damp by lambda_floor, and form the
    inverse square root and the square root (eigenvalues clamped at 0)."""
    A = np.asarray(A, dtype=np.float64)
    d = A.shape[0]
    if d % b:
        raise ValueError("d_in % b != 0")
    t, lam = trace_floor(A, eps)
    lam = max(lam, LAMBDA_MIN)
    S = np.zeros((d, b))
    S_inv = np.zeros((d, b))
    theta = np.zeros(d)
    for i in range(d // b):
        sl = slice(i * b, (i + 1) * b)
        w, V = np.linalg.eigh(A[sl, sl])
        w = np.maximum(w, 0.0)
        S[sl] = (V * (w + lam) ** -0.5) @ V.T
        S_inv[sl] = (V * (w + lam) ** 0.5) @ V.T
        theta[sl] = w[::-1]
    return BlockFactor(S=S, S_inv=S_inv, theta=theta, lambda_iso=lam, trace=t)


def block_apply(G, M):
    """G [:, block i] M_i for every block, M stacked as in BlockFactor."""
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    b = M.shape[1]
    out = np.empty_like(G)
    for i in range(G.shape[1] // b):
        sl = slice(i * b, (i + 1) * b)
        out[:, sl] = G[:, sl] @ M[sl]
    return out


def block_whiten(G, bf):
    return block_apply(G, bf.S)


def block_unwhiten(W, bf):
    return block_apply(W, bf.S_inv)


def block_roundtrip(G, bf, block128=False):
    """block-A: whiten -> fl32 -> quantize -> dequantize -> un-whiten.
    Returns (codes, inv, W32, G^ fp64, flags)."""
    W32 = block_whiten(G, bf).astype(np.float32)
    codes, inv, flags = quantize(W32, block128)
    What = dequantize(codes, inv, block128)
    return codes, inv, W32, block_unwhiten(What, bf), flags


# --------------------------------------------------------------------------
# full-rank and two-sided references (step 11)
# --------------------------------------------------------------------------

def _damped(M, eps):
    M = np.asarray(M, dtype=np.float64)
    lam = max(eps * np.trace(M) / M.shape[0], LAMBDA_MIN)
    return M + lam * np.eye(M.shape[0])


def sym_pair(M, eps=DAMP_EPS):
    """((M + lam I)^{-1/2}, (M + lam I)^{1/2}), lam = eps tr(M) / n, by eigh."""
    w, V = np.linalg.eigh(_damped(M, eps))
    w = np.maximum(w, 0.0)
    return (V * w ** -0.5) @ V.T, (V * w ** 0.5) @ V.T


def cholesky_pair(A, eps=DAMP_EPS):
    """(L^-T, L^T) with L L^T = A + lam I (L lower triangular)."""
    L = np.linalg.cholesky(_damped(A, eps))
    Linv = np.linalg.solve(L, np.eye(L.shape[0]))
    return Linv.T, L.T


def output_factor(G):
    """Output-side factor read as the gradient's row second moment G G^T / d_in."""
    G = np.asarray(G, dtype=np.float64)
    return G @ G.T / G.shape[1]


def reference_transforms(G, A, eps=DAMP_EPS):
    """{name: (left, right, left_inv, right_inv)} of the references; None
    stands for the identity."""
    S, Si = sym_pair(A, eps)
    Lt_inv, Lt = cholesky_pair(A, eps)
    SB, SBi = sym_pair(output_factor(G), eps)
    return {"input_full": (None, S, None, Si),
            "input_cholesky": (None, Lt_inv, None, Lt),
            "two_sided": (SB, S, SBi, Si)}


def _lr(M, left, right):
    M = np.asarray(M, dtype=np.float64)
    if left is not None:
        M = left @ M
    return M @ right if right is not None else M


def reference_roundtrip(G, transform, block128=False):
    """W = left G right -> fl32 -> quantize -> dequantize -> left_inv W^ right_inv.
    Returns (codes, inv, W32, G^ fp64)."""
    left, right, left_inv, right_inv = transform
    W32 = _lr(G, left, right).astype(np.float32)
    codes, inv, _ = quantize(W32, block128)
    return codes, inv, W32, _lr(dequantize(codes, inv, block128), left_inv, right_inv)


def reduce_payloads(payloads):
    """fp32 sum of dequantized payloads in the given order (step 8):
    S = D_0, then S = fl32(S + D_r).  payloads: list of (fmt, codes, scales)
    with fmt "tensor", "block128" or "mxfp4"."""
    S = None
    for fmt, codes, scales in payloads:
        if fmt == "mxfp4":
            D = mxfp4.dequantize(codes, scales)
        else:
            D = dequantize(codes, scales, fmt == "block128")
        D = np.asarray(D, dtype=np.float32)
        S = D.copy() if S is None else (S + D).astype(np.float32)
    return S


# --------------------------------------------------------------------------
# error metrics
# --------------------------------------------------------------------------

def error_sums(G, G_hat):
    """(sum (G^ - G)^2, sum G^2) in fp64."""
    G = np.asarray(G, dtype=np.float64)
    E = np.asarray(G_hat, dtype=np.float64) - G
    return float(np.sum(E * E)), float(np.sum(G * G))


def rel_frobenius(G, G_hat):
    """M1 = ||G^ - G||_F / ||G||_F (plain relative reconstruction error)."""
    e, g = error_sums(G, G_hat)
    return float(np.sqrt(e / g)) if g > 0 else float("nan")


def metric_sqrt_inv(A, lam):
    """(A + lam I)^{-1/2} by a full symmetric eigendecomposition (fp64)."""
    w, V = np.linalg.eigh(np.asarray(A, dtype=np.float64))
    return (V * (np.maximum(w, 0.0) + lam) ** -0.5) @ V.T


def rel_error_kfac(G, G_hat, S):
    """M2 = ||(G^ - G) S||_F / ||G S||_F with S = (A + lambda_floor I)^{-1/2}:
    the reconstruction error measured in the input-side K-FAC metric (GIFT
    review, axiom ledger: the Fisher information is the local metric)."""
    G = np.asarray(G, dtype=np.float64)
    E = np.asarray(G_hat, dtype=np.float64) - G
    return float(np.linalg.norm(E @ S) / np.linalg.norm(G @ S))


# --------------------------------------------------------------------------
# selective deployment
# --------------------------------------------------------------------------

def anisotropy(f):
    """rho = theta_1 / tr(A) of a factor: the share of the input's second
    moment in its leading direction (reading of the pages' "numerically
    vulnerable" layers, GIFT review referee report major comment 3)."""
    return float(f.theta[0]) / f.trace if f.trace > 0 else 0.0


def select_top_k(rhos, k):
    """Indices (ascending) of the k layers with the largest rho; None marks a
    layer that is never whitened; equal rho goes to the lower index."""
    eligible = [i for i, r in enumerate(rhos) if r is not None]
    chosen = []
    for _ in range(min(max(k, 0), len(eligible))):
        best = None
        for i in eligible:
            if i in chosen:
                continue
            if best is None or rhos[i] > rhos[best]:
                best = i
        chosen.append(best)
    return sorted(chosen)
