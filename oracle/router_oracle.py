"""Plain fp64 CPU oracle for the fused RMSNorm + MoE router top-K.

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's CPU-baseline leg
may import or run this module; the GPU library never calls it and shares no
code with it.

What it computes is read off the "RMSNorm Router Top-K A2AV Kernel API
Reference" page (awsdocs-neuron, nkilib experimental moe_block): the
"Background" section, the "API Reference" parameter and return list and its
"Notes" (the ACT2 pipeline).  The single-device part only: the normalised
hidden states, the top-K expert indices and the masked affinities.  The page
prints no numeric example; tests/test_router_oracle.py pins every function by
hand-computed closed forms, invariants and brute force.

Readings taken where the page is silent (each listed with the design notes):
  * RMSNorm is ``x / sqrt(mean(x^2) + eps) * gamma``, as on the attention page;
  * the router consumes the normalised states (the fusion the title names),
    before any rounding: logits = x_hat @ router_weights (+ router_bias);
  * the bias, when given, is part of the raw logits that top-K ranks and that
    the activation then sees;
  * top-K returns the K largest logits in descending order; among equal
    logits the lower expert index comes first;
  * SOFTMAX is taken over the K selected logits only, SIGMOID per selected
    logit; the affinities are not renormalised;
  * unselected experts hold exactly zero in the masked affinities.

Everything is in float64 on the exact input values (bf16 widened).
"""
import numpy as np

SIGMOID = 0
SOFTMAX = 1


def rms_norm_rows(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Per row: x / sqrt(mean(x^2) + eps) * gamma ("Background": the RMSNorm half)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64).reshape(1, -1)


def router_logits(x_hat: np.ndarray, w: np.ndarray, bias=None) -> np.ndarray:
    """Raw router logits [T, E] = x_hat @ router_weights (+ bias) ("API Reference":
    router_weights [H, E], router_bias [1, E])."""
    z = np.asarray(x_hat, dtype=np.float64) @ np.asarray(w, dtype=np.float64)
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64).reshape(1, -1)
    return z


def top_k(logits_row: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest values, descending; ties to the lower index
    ("Notes": top-K on the raw logits)."""
    z = np.asarray(logits_row, dtype=np.float64)
    order = sorted(range(z.shape[0]), key=lambda e: (-z[e], e))
    return np.asarray(order[:k], dtype=np.int64)


def activate_selected(sel_logits: np.ndarray, act: int) -> np.ndarray:
    """Activation on the selected logits only ("Notes": the ACT2 pipeline)."""
    z = np.asarray(sel_logits, dtype=np.float64)
    if act == SIGMOID:
        return 1.0 / (1.0 + np.exp(-z))
    if act == SOFTMAX:
        e = np.exp(z - np.max(z))
        return e / np.sum(e)
    raise ValueError(f"unknown activation {act}")


def rmsnorm_router_topk(hidden: np.ndarray, gamma: np.ndarray, w: np.ndarray, bias, eps: float, k: int, act: int):
    """The three returns of the page's function for [T, H] hidden states:
    (normalised states [T, H], indices [T, K] int64, masked affinities [T, E])."""
    x_hat = rms_norm_rows(hidden, gamma, eps)
    z = router_logits(x_hat, w, bias)
    T, E = z.shape
    idx = np.empty((T, k), dtype=np.int64)
    aff = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        sel = top_k(z[t], k)
        idx[t] = sel
        aff[t, sel] = activate_selected(z[t, sel], act)
    return x_hat, idx, aff
