"""fp64 CPU oracle: fused linear + Jensen-Shannon distillation loss, forward and backward.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it; the HIP product path never imports, links or calls
anything here, and nothing here imports the product.

Source (web page, cited by title and section):
  [distill] "perf(distillation): skip dW/dB calculation when parameters are frozen",
            Summary: a fused linear distillation loss (student and teacher heads over
            chunks of tokens, a JSD loss between their distributions) differentiates
            the student head's weight and bias on every chunk; when they do not
            require gradients, no gradient buffer is allocated and no per-chunk weight
            gradient product runs; when nothing requires gradients only the forward
            runs.  Details: B*T = 4096 tokens, H = 4096, V = 128256 / 151936, chunks of
            1024 tokens, bf16; loss and input gradients are unchanged by the skipping.

The page names the loss but prints no formula.  The readings taken (the textbook
weighted Jensen-Shannon divergence; they are the definition this oracle writes out):
  * logits: z_s = x_s W_s^T (+ b_s) and z_t = x_t W_t^T (+ b_t), one row per token;
  * distributions over the V classes at temperature tau: S = softmax(z_s / tau)
    (student), T = softmax(z_t / tau) (teacher);
  * per token, with mixture weight beta in [0, 1]:
        J = beta * KL(T || M) + (1 - beta) * KL(S || M),   M = beta * T + (1 - beta) * S,
    natural logarithms; beta = 0.5 is the symmetric JSD (bounded by ln 2);
  * the loss is the mean of J over the tokens; no hard-label term;
  * gradients flow to the student only (the teacher is a fixed target): input x_s,
    weight W_s and bias b_s, each skipped when not requested.

Everything is computed in float64 from the exact values of the (bf16) inputs, one
step after another; numpy's matmul serves as the matrix product.  Log-softmax is
taken as z - max(z) - log(sum(exp(z - max(z)))), the usual exact rewriting.
"""
from __future__ import annotations

import numpy as np

__all__ = ["log_softmax", "jsd_rows", "fused_linear_jsd"]


def log_softmax(z: np.ndarray) -> np.ndarray:
    """Row-wise log-softmax of a 2-D fp64 array."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=1, keepdims=True)
    return z - m - np.log(np.exp(z - m).sum(axis=1, keepdims=True))


def jsd_rows(zs: np.ndarray, zt: np.ndarray, beta: float, temperature: float):
    """Per-token weighted JSD between student and teacher logits, and its gradient with
    respect to the student logits.

    Returns (J [rows], dJ/dz_s [rows, V]).  With g_v = dJ/dS_v = (1 - beta) *
    log(S_v / M_v) (the teacher terms do not depend on S, and the two "+1"s of the
    derivative of S log S - M log M cancel), the softmax backward at temperature tau
    gives dJ/dz_v = S_v * (g_v - sum_u S_u g_u) / tau."""
    tau = float(temperature)
    b = float(beta)
    ls = log_softmax(np.asarray(zs, np.float64) / tau)
    lt = log_softmax(np.asarray(zt, np.float64) / tau)
    s, t = np.exp(ls), np.exp(lt)
    m = b * t + (1.0 - b) * s
    with np.errstate(divide="ignore", invalid="ignore"):
        lm = np.log(m)
        # terms with a zero weight contribute 0 (0 * log 0 = 0)
        kl_t = np.where(t > 0, t * (lt - lm), 0.0).sum(axis=1)
        kl_s = np.where(s > 0, s * (ls - lm), 0.0).sum(axis=1)
        g = np.where(s > 0, (1.0 - b) * (ls - lm), 0.0)
    j = b * kl_t + (1.0 - b) * kl_s
    dz = s * (g - (s * g).sum(axis=1, keepdims=True)) / tau
    return j, dz


def fused_linear_jsd(xs, ws, bs, xt, wt, bt, beta: float = 0.5, temperature: float = 1.0,
                     need_dx: bool = True, need_dw: bool = True, need_db: bool = True):
    """Loss and student gradients of the fused linear JSD distillation loss.

    xs [BT, H], ws [V, H], bs [V] or None; xt [BT, Ht], wt [V, Ht], bt [V] or None.
    Returns a dict: loss (scalar), per_token J [BT], zs, zt (logits), dz (dL/dz_s),
    and dx [BT, H], dw [V, H], db [V] for the gradients requested (None otherwise)."""
    xs = np.asarray(xs, np.float64)
    ws = np.asarray(ws, np.float64)
    xt = np.asarray(xt, np.float64)
    wt = np.asarray(wt, np.float64)
    bt_tokens = xs.shape[0]
    zs = xs @ ws.T
    if bs is not None:
        zs = zs + np.asarray(bs, np.float64)[None, :]
    zt = xt @ wt.T
    if bt is not None:
        zt = zt + np.asarray(bt, np.float64)[None, :]
    j, dj = jsd_rows(zs, zt, beta, temperature)
    loss = j.sum() / bt_tokens if bt_tokens else 0.0
    dz = dj / bt_tokens if bt_tokens else dj
    out = {"loss": loss, "per_token": j, "zs": zs, "zt": zt, "dz": dz,
           "dx": None, "dw": None, "db": None}
    if need_dx:
        out["dx"] = dz @ ws
    if need_dw:
        out["dw"] = dz.T @ xs
    if need_db and bs is not None:
        out["db"] = dz.sum(axis=0)
    return out
