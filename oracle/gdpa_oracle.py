"""fp64 CPU oracle for Generalized Dot-Product Attention (GDPA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes (Kunlun paper summary, section 2.2 "low-level module
optimisations", GDPA bullet; Telegram review of the same paper, layer steps 1
and 2): the personalised FFN recast as one multi-head attention operator.  The
tokens of a sample's user history are the queries; the keys and values are
per-sample weights derived from that sample's non-sequential context.  For a
jagged batch with sample b owning rows offsets[b]:offsets[b+1] of Q[T,H,d] and
per-sample K[b], V[b] of shape [n,H,d], per head h:

    S = scale * X Kb^T            (X = Q rows of b, head h; Kb = K[b,:,h,:])
    P = phi(S)                    (row softmax over the n context rows, or elementwise)
    O = P Vb

The pages give no formula for the score map, the scale, masking or the
normalisation.  Readings taken (each listed with its reason in the design notes):
  * phi is a row softmax over the sample's n rows, or an elementwise map: SiLU
    s*sigmoid(s) (the FFN form silu(x K^T) V), ReLU max(s, 0) (derivative 0 at
    s = 0), GELU s*Phi(s) with Phi the standard normal CDF (the exact erf form),
    or the identity (then GDPA is the bilinear map (x K^T) V);
  * scale defaults to 1/sqrt(d) for softmax and 1.0 for the elementwise maps;
  * no mask: each token sees all n rows of its own sample and nothing else;
  * d_v = d_qk = d, K and V are distinct per head;
  * no FFN bias.

Everything is plain float64 numpy: a matrix product is the only library step.
No blocking, no online softmax, no fusion.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np
from scipy.special import erf as _erf

PHIS = ("softmax", "silu", "relu", "gelu", "identity")


def as_f64(x) -> np.ndarray:
    """float64 numpy copy of a numpy array or a (CPU or device) torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        try:
            import torch  # local: only to widen bf16, which numpy cannot hold
            x = x.to(torch.float64)
        except ImportError:  # pragma: no cover
            pass
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def default_scale(phi: str, d: int) -> float:
    """1/sqrt(d) for softmax (standard attention), 1.0 for the elementwise maps (the plain
    FFN form)."""
    if phi == "softmax":
        return 1.0 / math.sqrt(d)
    if phi in PHIS:
        return 1.0
    raise ValueError(f"phi must be one of {PHIS}, got {phi!r}")


def sigmoid(s: np.ndarray) -> np.ndarray:
    """Logistic function, evaluated without overflow on either side."""
    out = np.empty_like(s)
    pos = s >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-s[pos]))
    e = np.exp(s[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(s: np.ndarray) -> np.ndarray:
    """SiLU(s) = s * sigmoid(s)."""
    return s * sigmoid(s)


def silu_grad(s: np.ndarray) -> np.ndarray:
    """d/ds [s sigmoid(s)] = sigmoid(s) (1 + s (1 - sigmoid(s)))."""
    g = sigmoid(s)
    return g * (1.0 + s * (1.0 - g))


def relu(s: np.ndarray) -> np.ndarray:
    """max(s, 0)."""
    return np.maximum(s, 0.0)


def relu_grad(s: np.ndarray) -> np.ndarray:
    """1 for s > 0, else 0 (the subgradient 0 is taken at s = 0)."""
    return (s > 0).astype(np.float64)


def normal_cdf(s: np.ndarray) -> np.ndarray:
    """Phi(s) = (1 + erf(s / sqrt 2)) / 2."""
    return 0.5 * (1.0 + _erf(s / math.sqrt(2.0)))


def gelu(s: np.ndarray) -> np.ndarray:
    """GELU(s) = s Phi(s) (the exact form, not the tanh approximation)."""
    return s * normal_cdf(s)


def gelu_grad(s: np.ndarray) -> np.ndarray:
    """d/ds [s Phi(s)] = Phi(s) + s exp(-s^2 / 2) / sqrt(2 pi)."""
    return normal_cdf(s) + s * np.exp(-0.5 * s * s) / math.sqrt(2.0 * math.pi)


# Elementwise score maps: (value, derivative), looked up by name at call time.
ELEMENTWISE = {
    "silu": (lambda s: silu(s), lambda s: silu_grad(s)),
    "relu": (lambda s: relu(s), lambda s: relu_grad(s)),
    "gelu": (lambda s: gelu(s), lambda s: gelu_grad(s)),
    "identity": (lambda s: s, lambda s: np.ones_like(s)),
}


def row_softmax(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax over the last axis and its log-sum-exp (natural log)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


# ---------------------------------------------------------------------------
# One (sample, head) pair: the definition itself.
# ---------------------------------------------------------------------------

def gdpa_forward_bh(x: np.ndarray, kb: np.ndarray, vb: np.ndarray, phi: str,
                    scale: float, sbias=None, obias=None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """O = phi(scale * x kb^T [+ sbias]) vb [+ obias] for one sample and head.

    x: [L, d] query rows, kb, vb: [n, d]; sbias [n] (one per context row, the
    FFN's hidden bias), obias [d] (the FFN's output bias).  Returns (O [L, d],
    lse [L] or None).
    """
    s = scale * (x @ kb.T)                      # [L, n]
    if sbias is not None:
        s = s + sbias[None, :]
    if phi == "softmax":
        p, lse = row_softmax(s)
        o = p @ vb
    elif phi in ELEMENTWISE:
        o, lse = ELEMENTWISE[phi][0](s) @ vb, None
    else:
        raise ValueError(phi)
    if obias is not None:
        o = o + obias[None, :]
    return o, lse


def gdpa_backward_bh(x: np.ndarray, kb: np.ndarray, vb: np.ndarray, do: np.ndarray,
                     phi: str, scale: float, sbias=None, with_bias_grads: bool = False):
    """Gradients of sum(O * dO) w.r.t. x, kb, vb (and the biases) for one sample and head.

    Chain rule through O = P V + obias, P = phi(S), S = scale x kb^T + sbias:
      dV = P^T dO;  dP = dO V^T;
      softmax: dS = P * (dP - rowsum(dO * (P V)));  elementwise: dS = dP * phi'(S);
      dX = scale dS kb;  dK = scale dS^T x;  dsbias = column sums of dS;
      dobias = column sums of dO.
    """
    s = scale * (x @ kb.T)
    if sbias is not None:
        s = s + sbias[None, :]
    dp = do @ vb.T
    if phi == "softmax":
        p, _ = row_softmax(s)
        o = p @ vb
        dvec = (do * o).sum(axis=-1, keepdims=True)
        ds = p * (dp - dvec)
    elif phi in ELEMENTWISE:
        f, fg = ELEMENTWISE[phi]
        p = f(s)
        ds = dp * fg(s)
    else:
        raise ValueError(phi)
    dv = p.T @ do
    dx = scale * (ds @ kb)
    dk = scale * (ds.T @ x)
    if with_bias_grads:
        return dx, dk, dv, ds.sum(axis=0), do.sum(axis=0)
    return dx, dk, dv


# ---------------------------------------------------------------------------
# Jagged batch.
# ---------------------------------------------------------------------------

def _check(q, offsets, k, v):
    T, H, d = q.shape
    B, n, Hk, dk_ = k.shape
    if v.shape != k.shape or Hk != H or dk_ != d:
        raise ValueError("shape mismatch between Q [T,H,d] and K/V [B,n,H,d]")
    if len(offsets) != B + 1 or offsets[0] != 0 or offsets[-1] != T:
        raise ValueError("offsets must have B+1 entries from 0 to T")
    if np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must be non-decreasing")
    return T, H, d, B, n


def _check_jagged(q, offsets, kv_offsets, k, v):
    """Jagged context: k, v [rows,H,d], sample b owns rows kv_offsets[b]:kv_offsets[b+1], at least one."""
    T, H, d = q.shape
    B = len(offsets) - 1
    if k.ndim != 3 or v.shape != k.shape or k.shape[1:] != (H, d):
        raise ValueError("jagged K/V must be [rows,H,d] with the heads and width of Q")
    if len(kv_offsets) != B + 1 or kv_offsets[0] != 0 or kv_offsets[-1] != k.shape[0]:
        raise ValueError("kv_offsets must have B+1 entries from 0 to the number of rows")
    if np.any(np.diff(kv_offsets) < 1):
        raise ValueError("every sample needs at least one context row")
    if offsets[0] != 0 or offsets[-1] != T or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must be non-decreasing from 0 to T")
    return T, H, d, B


def _context(k, v, b, h, kv_offsets):
    """K and V rows of sample b, head h: the dense [B,n,H,d] slice or the jagged rows."""
    if kv_offsets is None:
        return k[b, :, h, :], v[b, :, h, :]
    r = slice(int(kv_offsets[b]), int(kv_offsets[b + 1]))
    return k[r, h, :], v[r, h, :]


def _score_bias(sb, b, h, kv_offsets):
    """Score bias of sample b, head h: [B,n,H] dense or [rows,H] jagged, or None."""
    if sb is None:
        return None
    if kv_offsets is None:
        return sb[b, :, h]
    return sb[int(kv_offsets[b]):int(kv_offsets[b + 1]), h]


def gdpa_forward(q, offsets, k, v, phi: str = "softmax", scale: Optional[float] = None,
                 samples: Optional[Sequence[int]] = None, kv_offsets=None, score_bias=None,
                 out_bias=None):
    """Forward over a jagged batch.

    q: [T,H,d]; offsets: [B+1]; k, v: [B,n,H,d], or with kv_offsets [B+1] a jagged
    context [rows,H,d] (sample b owns rows kv_offsets[b]:kv_offsets[b+1]).  Returns
    (O [T,H,d], lse [T,H] for softmax else None), float64.  With `samples`, only
    those samples' rows are computed (the rest stay NaN): samples are independent.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    offsets = np.asarray(as_f64(offsets), dtype=np.int64)
    if kv_offsets is None:
        T, H, d, B, n = _check(q, offsets, k, v)
    else:
        kv_offsets = np.asarray(as_f64(kv_offsets), dtype=np.int64)
        T, H, d, B = _check_jagged(q, offsets, kv_offsets, k, v)
    sb = None if score_bias is None else as_f64(score_bias)    # [B,n,H] or [rows,H]
    ob = None if out_bias is None else as_f64(out_bias)        # [B,H,d]
    if scale is None:
        scale = default_scale(phi, d)
    o = np.full((T, H, d), np.nan)
    lse = np.full((T, H), np.nan) if phi == "softmax" else None
    for b in (range(B) if samples is None else samples):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        for h in range(H):
            kb, vb = _context(k, v, b, h, kv_offsets)
            ohb, lb = gdpa_forward_bh(q[r0:r1, h, :], kb, vb, phi, scale, _score_bias(sb, b, h, kv_offsets),
                                      None if ob is None else ob[b, h])
            o[r0:r1, h, :] = ohb
            if lse is not None:
                lse[r0:r1, h] = lb
    return o, lse


def gdpa_backward(q, offsets, k, v, do, phi: str = "softmax", scale: Optional[float] = None,
                  samples: Optional[Sequence[int]] = None, kv_offsets=None, score_bias=None,
                  bias_grads: bool = False):
    """Backward over a jagged batch: (dQ [T,H,d], dK, dV shaped like K, V), and with
    bias_grads also (d score_bias shaped like K without d, d out_bias [B,H,d]).

    dK, dV and the bias gradients are sums over each sample's own tokens; an
    empty sample gets zeros.  With `samples`, other samples' slots stay NaN.
    """
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    offsets = np.asarray(as_f64(offsets), dtype=np.int64)
    if kv_offsets is None:
        T, H, d, B, n = _check(q, offsets, k, v)
    else:
        kv_offsets = np.asarray(as_f64(kv_offsets), dtype=np.int64)
        T, H, d, B = _check_jagged(q, offsets, kv_offsets, k, v)
    if scale is None:
        scale = default_scale(phi, d)
    sb = None if score_bias is None else as_f64(score_bias)
    dq = np.full((T, H, d), np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    dsb = np.full(k.shape[:-1], np.nan)
    dob = np.full((B, H, d), np.nan)
    for b in (range(B) if samples is None else samples):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        for h in range(H):
            kb, vb = _context(k, v, b, h, kv_offsets)
            gx, gk, gv, gsb, gob = gdpa_backward_bh(q[r0:r1, h, :], kb, vb, do[r0:r1, h, :], phi, scale,
                                                    _score_bias(sb, b, h, kv_offsets), with_bias_grads=True)
            dq[r0:r1, h, :] = gx
            dob[b, h] = gob
            if kv_offsets is None:
                dk[b, :, h, :] = gk
                dv[b, :, h, :] = gv
                dsb[b, :, h] = gsb
            else:
                c = slice(int(kv_offsets[b]), int(kv_offsets[b + 1]))
                dk[c, h, :] = gk
                dv[c, h, :] = gv
                dsb[c, h] = gsb
    if bias_grads:
        return dq, dk, dv, dsb, dob
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Stacked residual layers with generated K/V (Telegram review, layer step 1:
# K and V come from the context features; paper summary section 2.1: the
# weight-generation module of the interaction block; section 2.2, GDPA bullet:
# the personalised FFN becomes stable to stack, read as a plain residual between
# layers).
# ---------------------------------------------------------------------------

def weight_generation(ctx, w, n: int, H: int, d: int) -> np.ndarray:
    """K (or V) = (C W^T).reshape(B, n, H, d) for context C [B, c] and an
    output-major weight W [n*H*d, c] (a linear layer's weight layout)."""
    ctx, w = as_f64(ctx), as_f64(w)
    return (ctx @ w.T).reshape(ctx.shape[0], n, H, d)


def weight_gradient(ctx, d_out) -> np.ndarray:
    """dW [cols, c] = d_out[B, cols]^T C[B, c]: gradient of C W^T with respect to W."""
    return as_f64(d_out).T @ as_f64(ctx)


def stacked_forward(x0, offsets, ctx, w_k: List, w_v: List, heads: int, n: int,
                    phi: str = "silu", scale: Optional[float] = None):
    """X_{l+1} = X_l + GDPA(X_l as [T,H,d]; C W_K^l, C W_V^l).  Returns [X_0..X_L] ([T,H*d])."""
    x = as_f64(x0)
    T, HD = x.shape
    d = HD // heads
    xs = [x]
    for wk, wv in zip(w_k, w_v):
        kl = weight_generation(ctx, wk, n, heads, d)
        vl = weight_generation(ctx, wv, n, heads, d)
        o, _ = gdpa_forward(x.reshape(T, heads, d), offsets, kl, vl, phi, scale)
        x = x + o.reshape(T, HD)
        xs.append(x)
    return xs


def stacked_backward(xs: List[np.ndarray], offsets, ctx, w_k: List, w_v: List, do,
                     heads: int, n: int, phi: str = "silu", scale: Optional[float] = None):
    """Backward of stacked_forward for loss sum(X_L * dO).

    dX_l = dX_{l+1} + dQ_l (the residual passes the gradient through unchanged);
    dW^l = dK_l.reshape(B, -1)^T C (and likewise for V), in W's [n*H*d, c] layout.
    Returns (dX_0, [dW_K], [dW_V]).
    """
    ctx = as_f64(ctx)
    dx = as_f64(do)
    T, HD = dx.shape
    d = HD // heads
    B = ctx.shape[0]
    dwk = [None] * len(w_k)
    dwv = [None] * len(w_v)
    for l in reversed(range(len(w_k))):
        kl = weight_generation(ctx, w_k[l], n, heads, d)
        vl = weight_generation(ctx, w_v[l], n, heads, d)
        gq, gk, gv = gdpa_backward(xs[l].reshape(T, heads, d), offsets, kl, vl,
                                   dx.reshape(T, heads, d), phi, scale)
        dwk[l] = gk.reshape(B, -1).T @ ctx
        dwv[l] = gv.reshape(B, -1).T @ ctx
        dx = dx + gq.reshape(T, HD)
    return dx, dwk, dwv
