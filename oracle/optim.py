"""Plain fp64 numpy implementation of the optimiser step that follows the
backward pass: AdamW on the embedding and unembedding, Muon on every block
matrix, a linear-to-zero learning-rate multiplier, and gradient
accumulation over micro-batches.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product never
imports this module.

What the pages state (nanochat speedrun walkthrough, lyylswood.com, "100
dollars, 8000 lines: a hand-built ChatGPT clone", section Pretraining):

* the matrices are optimised with Muon and the embedding and unembedding
  with AdamW; no other tensor is trainable (optimiser paragraph);
* learning rates are scaled as 1/sqrt(model width) (learning-rate
  paragraph);
* the logged lrm is a learning-rate multiplier that falls linearly to 0
  near the end of training (the paragraph after the training log);
* one optimiser step consumes 32 x 2048 tokens per GPU on 8 GPUs
  (2^19 tokens), so one GPU reaches that batch by accumulating gradients
  over micro-batches (the launch paragraph).

The pages name Muon without defining it.  This module follows the
published definition (K. Jordan et al., "Muon: An optimizer for hidden
layers in neural networks", 2024): heavy-ball momentum with a Nesterov
look-ahead, whose update direction is replaced by an approximate
orthogonalisation from five steps of a quintic Newton-Schulz iteration on
the Frobenius-normalised direction, X <- a X + (b A + c A^2) X with
A = X X^T and (a, b, c) = (3.4445, -4.7750, 2.0315), iterated on the wide
orientation (a tall matrix is transposed first and back after), and the
step scaled by sqrt(max(1, rows / cols)).  AdamW is the decoupled-decay
form of Loshchilov and Hutter ("Decoupled Weight Decay Regularization",
2019) with bias-corrected moments.

Readings where the pages are silent (listed in the design notes): the
hyperparameter defaults of ``default_hparams``; q, k and v are three
separate matrices for Muon although they are stored as one [3d, d] block;
the schedule's warm-down is the last 20 % of the iterations; gradients
accumulated over n micro-batches are averaged (grad_scale = 1/n).

Everything is fp64 and written step by step from those definitions, with
numpy's matmul as the only library primitive.
"""
from __future__ import annotations

import math
import numpy as np

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_EPS = 1e-7


# ---------------------------------------------------------------------------
# AdamW (decoupled weight decay, bias-corrected moments)
# ---------------------------------------------------------------------------
def adamw_update(p, g, m, v, step, lr, beta1, beta2, eps, wd):
    """One AdamW step on arrays of any shape; step is 1-based.

    p <- p (1 - lr wd);  m <- beta1 m + (1 - beta1) g;
    v <- beta2 v + (1 - beta2) g^2;
    p <- p - lr (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps).
    Returns the new (p, m, v)."""
    p = p * (1.0 - lr * wd)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


# ---------------------------------------------------------------------------
# Muon
# ---------------------------------------------------------------------------
def newton_schulz(G, steps=5, coeffs=NS_COEFFS, eps=NS_EPS):
    """Approximate orthogonalisation of a matrix: X = G / (||G||_F + eps),
    on the wide orientation (rows <= cols; a tall G is transposed first and
    the result transposed back), then `steps` times
    A = X X^T;  B = b A + c A A;  X = a X + B X."""
    a, b, c = coeffs
    tall = G.shape[0] > G.shape[1]
    X = G.T if tall else G
    X = X / (np.linalg.norm(X) + eps)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if tall else X


def muon_update(W, G, buf, lr, momentum, nesterov=True, ns_steps=5, coeffs=NS_COEFFS, eps=NS_EPS):
    """One Muon step on a matrix W [rows, cols] with gradient G and momentum
    buffer buf (zeros before the first step).

    buf <- momentum buf + G;  u = G + momentum buf (Nesterov) or buf;
    W <- W - lr sqrt(max(1, rows / cols)) newton_schulz(u).
    Returns the new (W, buf)."""
    buf = momentum * buf + G
    u = G + momentum * buf if nesterov else buf
    O = newton_schulz(u, ns_steps, coeffs, eps)
    scale = math.sqrt(max(1.0, W.shape[0] / W.shape[1]))
    return W - lr * scale * O, buf


# ---------------------------------------------------------------------------
# schedule
# ---------------------------------------------------------------------------
def lr_multiplier(it, num_iters, warmdown_ratio=0.2, final_frac=0.0):
    """1 until the last warmdown_ratio of the iterations, then linear down
    to final_frac at it = num_iters."""
    progress = it / num_iters
    if progress < 1.0 - warmdown_ratio:
        return 1.0
    return final_frac + (1.0 - final_frac) * (1.0 - progress) / warmdown_ratio


def muon_momentum(it, start=0.85, end=0.95, ramp_iters=300):
    """Momentum raised linearly from start to end over the first
    ramp_iters steps."""
    frac = min(it / ramp_iters, 1.0)
    return (1.0 - frac) * start + frac * end


def default_hparams(d_model, it, num_iters, n_micro=1):
    """The step's hyperparameters (readings; every value can be overridden).
    AdamW learning rates carry the 1/sqrt(width) scale, taken relative to a
    768-wide model; lrm multiplies every learning rate."""
    lrm = lr_multiplier(it, num_iters)
    width_scale = (d_model / 768.0) ** -0.5
    return {
        "grad_scale": 1.0 / n_micro,
        "lr_embed": 0.2 * width_scale * lrm,
        "lr_unembed": 0.004 * width_scale * lrm,
        "beta1": 0.8, "beta2": 0.95, "eps": 1e-10, "weight_decay": 0.0,
        "adam_step": it + 1,
        "lr_matrix": 0.02 * lrm,
        "momentum": muon_momentum(it),
        "nesterov": True, "ns_steps": 5, "ns_coeffs": NS_COEFFS,
    }


# ---------------------------------------------------------------------------
# the whole step over the flat parameter buffer
# ---------------------------------------------------------------------------
def new_state(layout):
    """Zero optimiser state for a parameter layout (list of (name, layer,
    rows, cols, offset)): AdamW moments for E and U, a momentum buffer for
    every matrix."""
    st = {}
    for name, layer, r, c, off in layout:
        if name in ("E", "U"):
            st[(name, layer, "m")] = np.zeros((r, c))
            st[(name, layer, "v")] = np.zeros((r, c))
        else:
            st[(name, layer, "buf")] = np.zeros((r, c))
    return st


def optimizer_step(layout, master, grads, state, hp):
    """One optimiser step.  master (fp64 flat parameters) and state are
    updated copies; grads is the flat gradient (a sum over micro-batches,
    scaled by hp["grad_scale"]).  Returns (master, state)."""
    master = master.copy()
    state = dict(state)
    for name, layer, r, c, off in layout:
        p = master[off:off + r * c].reshape(r, c)
        g = grads[off:off + r * c].reshape(r, c) * hp["grad_scale"]
        if name in ("E", "U"):
            lr = hp["lr_embed"] if name == "E" else hp["lr_unembed"]
            p, m, v = adamw_update(p, g, state[(name, layer, "m")], state[(name, layer, "v")], hp["adam_step"],
                                   lr, hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"])
            state[(name, layer, "m")], state[(name, layer, "v")] = m, v
        else:
            p, buf = muon_update(p, g, state[(name, layer, "buf")], hp["lr_matrix"], hp["momentum"],
                                 hp["nesterov"], hp["ns_steps"], hp["ns_coeffs"])
            state[(name, layer, "buf")] = buf
        master[off:off + r * c] = p.ravel()
    return master, state
