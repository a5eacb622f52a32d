"""Seeded synthetic activations, gradients and sketches.

Recipe (the same for every workload; only shapes, token counts and spectra
change):

* eigenbasis: Q = Haar-random orthogonal d x d (QR of a Gaussian matrix,
  columns sign-fixed by diag(R) > 0);
* spectrum: ev_i = i^-p, i = 1..d (power law, exponent p, default 1.5);
* activations: X = Z_X diag(ev^1/2) Q^T, Z_X an N x d standard Gaussian, so
  E[x x^T] = C = Q diag(ev) Q^T; cast to bf16 values where the workload
  says bf16 (kept in an fp32 tensor holding exactly bf16-representable
  values, or returned as a bf16 tensor);
* gradients: G = diag(s) Z_G diag(ev^1/2) Q^T with s_i = exp(N(0, 1)) per
  row (lognormal sigma = 1) and Z_G a d_out x d standard Gaussian.  This
  has the distribution of diag(s) Z C^1/2 (Z Q is again Gaussian), at the
  cost of one product with Q instead of two;
* sketches for device/oracle parity runs: a seeded d x l standard Gaussian.

Everything is drawn with a seeded torch.Generator on the requested device, in
a fixed order, so a (workload, seed, device) triple always gives the same
tensors.  This module performs none of the method's arithmetic.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import torch


@dataclass
class InputSpec:
    """One distinct layer input (one K-FAC factor)."""
    name: str
    d_in: int
    tokens: int
    exponent: float = 1.5
    bf16: bool = True


@dataclass
class LayerSpec:
    """One weight gradient G (d_out x d_in); input None => Euclidean-only layer
    with an isotropic Gaussian gradient (embedding / head)."""
    name: str
    d_out: int
    input: Optional[str]
    d_in: int = 0


@dataclass
class Workload:
    name: str
    inputs: List[InputSpec] = field(default_factory=list)
    layers: List[LayerSpec] = field(default_factory=list)

    def input(self, name):
        for s in self.inputs:
            if s.name == name:
                return s
        raise KeyError(name)

    @property
    def gradient_elements(self):
        return sum(l.d_out * l.d_in for l in self.layers)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def single_layer(d_in=512, d_out=256, tokens=4096, exponent=1.5, bf16=False):
    """One linear layer at CPU scale: d_in 512, d_out 256, 4096 fp32 tokens."""
    w = Workload("single_layer_%dx%d" % (d_out, d_in))
    w.inputs.append(InputSpec("x", d_in, tokens, exponent, bf16))
    w.layers.append(LayerSpec("w", d_out, "x", d_in))
    return w


def _block(w, prefix, hidden, mlp, tokens, exponents):
    e = list(exponents)
    ins = [InputSpec(prefix + "attn_in", hidden, tokens, e[0]),
           InputSpec(prefix + "o_in", hidden, tokens, e[1]),
           InputSpec(prefix + "mlp_in", hidden, tokens, e[2]),
           InputSpec(prefix + "down_in", mlp, tokens, e[3])]
    w.inputs.extend(ins)
    for name, d_out, inp in (("q", hidden, "attn_in"), ("k", hidden, "attn_in"),
                             ("v", hidden, "attn_in"), ("o", hidden, "o_in"),
                             ("gate", mlp, "mlp_in"), ("up", mlp, "mlp_in"),
                             ("down", hidden, "down_in")):
        d_in = mlp if inp == "down_in" else hidden
        w.layers.append(LayerSpec(prefix + name, d_out, prefix + inp, d_in))


def llama_block(hidden=1024, mlp=2816, tokens=8192, exponent=1.5):
    """One Llama-style block: q, k, v, o (hidden^2), gate/up (mlp x hidden),
    down (hidden x mlp); four distinct inputs (attention in, o in, MLP in,
    down in), each with its own eigenbasis."""
    w = Workload("llama_block_h%d_m%d_n%d" % (hidden, mlp, tokens))
    _block(w, "", hidden, mlp, tokens, [exponent] * 4)
    return w


def llama_stack(n_blocks=24, hidden=1024, mlp=2816, tokens=8192,
                exponent_range=None, exponent=1.5, vocab=0, seed=0):
    """n_blocks Llama-style blocks; optional vocab x hidden embedding and head
    gradients (Euclidean only).  exponent_range=(lo, hi) draws each input's
    spectral exponent uniformly (seeded), else every input uses `exponent`."""
    w = Workload("llama_stack_b%d_h%d_m%d_n%d" % (n_blocks, hidden, mlp, tokens))
    g = torch.Generator().manual_seed(10_000 + seed)
    for b in range(n_blocks):
        if exponent_range is None:
            ex = [exponent] * 4
        else:
            lo, hi = exponent_range
            ex = (lo + (hi - lo) * torch.rand(4, generator=g, dtype=torch.float64)).tolist()
        _block(w, "b%d." % b, hidden, mlp, tokens, ex)
    if vocab:
        w.layers.append(LayerSpec("embed", vocab, None, hidden))
        w.layers.append(LayerSpec("head", vocab, None, hidden))
    return w


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------

def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def haar(d, gen, device="cpu", dtype=torch.float32, host_qr=False):
    """Haar-random orthogonal d x d matrix (QR of a Gaussian, sign-fixed).

    host_qr: draw the Gaussian on `device` but factor it on the host (for
    runs under hardware-counter collection, which the device QR does not
    survive)."""
    z = torch.randn(d, d, generator=gen, device=device, dtype=torch.float64
                    if torch.device(device).type == "cpu" else torch.float32)
    if host_qr and torch.device(device).type != "cpu":
        q, r = torch.linalg.qr(z.cpu().double())
        q = q * torch.sign(torch.diagonal(r)).unsqueeze(0)
        return q.to(device=device, dtype=dtype)
    q, r = torch.linalg.qr(z)
    q = q * torch.sign(torch.diagonal(r)).unsqueeze(0)
    return q.to(dtype)


def power_law(d, exponent, device="cpu"):
    i = torch.arange(1, d + 1, device=device, dtype=torch.float64)
    return (i ** -exponent).to(torch.float32)


def to_bf16_values(x):
    """fp32 tensor holding exactly the bf16 (RNE) values of x."""
    return x.to(torch.bfloat16).to(torch.float32)


def draw_input(spec, seed, device="cpu", tokens=None, Q=None, as_bf16=False, host_qr=False,
               axis_aligned=False):
    """-> dict(Q, ev, X): eigenbasis, spectrum and N x d activations.

    X is fp32 (holding bf16 values when spec.bf16) unless as_bf16, which
    returns a bf16 tensor for bf16 inputs.  axis_aligned: the eigenbasis is
    the identity (Q is None), X = Z diag(ev^1/2) -- no QR, for runs under
    hardware-counter collection, where only the bytes moved matter.
    """
    n = spec.tokens if tokens is None else tokens
    g = _gen(seed, device)
    if Q is None and not axis_aligned:
        Q = haar(spec.d_in, g, device, host_qr=host_qr)
    ev = power_law(spec.d_in, spec.exponent, device)
    z = torch.randn(n, spec.d_in, generator=g, device=device, dtype=torch.float32)
    X = z * ev.sqrt()
    if Q is not None:
        X = X @ Q.T
    if spec.bf16:
        X = X.to(torch.bfloat16)
        if not as_bf16:
            X = X.to(torch.float32)
    return {"Q": Q, "ev": ev, "X": X}


def draw_gradient(d_out, Q, ev, seed, device="cpu"):
    """G = diag(s) Z diag(ev^1/2) Q^T, s lognormal(0, 1) per row; fp32 (Q None:
    the axis-aligned basis, no product)."""
    g = _gen(seed, device)
    d = ev.shape[0]
    s = torch.exp(torch.randn(d_out, generator=g, device=device, dtype=torch.float32))
    z = torch.randn(d_out, d, generator=g, device=device, dtype=torch.float32)
    G = z * ev.sqrt()
    if Q is not None:
        G = G @ Q.T
    return G * s.unsqueeze(1)


def draw_isotropic_gradient(d_out, d_in, seed, device="cpu"):
    """Gaussian gradient with lognormal row scales (embedding / head)."""
    g = _gen(seed, device)
    s = torch.exp(torch.randn(d_out, generator=g, device=device, dtype=torch.float32))
    z = torch.randn(d_out, d_in, generator=g, device=device, dtype=torch.float32)
    return z * s.unsqueeze(1)


def gaussian_sketch(d, width, seed, device="cpu"):
    """Seeded d x width standard Gaussian (fp32)."""
    g = _gen(seed, device)
    return torch.randn(d, width, generator=g, device=device, dtype=torch.float32)


def rotation_pair(d, seed, device="cpu"):
    """Haar basis V for a slowly rotating eigenbasis R(t) = V B(t phi) V^T,
    B = block-diagonal 2x2 plane rotations (every principal angle of R(t) is
    exactly t phi)."""
    return haar(d, _gen(seed, device), device)


def rotate_input(Q, V, angle):
    """R Q with R = V B(angle) V^T (d even: d/2 planes; odd d: last axis fixed)."""
    d = Q.shape[0]
    P = V.T @ Q
    c, s = torch.cos(torch.tensor(angle, dtype=torch.float64)), torch.sin(
        torch.tensor(angle, dtype=torch.float64))
    c, s = float(c), float(s)
    m = d - (d % 2)
    a = P[0:m:2].clone()
    b = P[1:m:2].clone()
    P = P.clone()
    P[0:m:2] = c * a - s * b
    P[1:m:2] = s * a + c * b
    return V @ P
