"""Recall head and gate, in float64 (oracle side).

ODA summary page, "Approach": the recall head takes three inputs available
before any global read -- the previously selected hidden state h_{t-1}, the
embedding of the current input token E(x_t), and the final hidden state of the
current Local pass h^L_t -- and returns one scalar q_t; the step recalls (reruns
with full attention) when q_t > theta, with theta = 0 by default. "Developer
perspective": the head is evaluated in FP32 on the GPU.

The pages give only the head's parameter count, not its layout. The head here is
a two-layer MLP over the concatenation [h_{t-1}, E(x_t), h^L_t] in that order:

    a   = W1 x + b1
    u   = GELU(a) = a * (1 + erf(a / sqrt 2)) / 2      (exact-erf GELU)
    q_t = <w2, u> + b2
"""

import math

import numpy as np
from scipy.special import erf


def concat_inputs(h_prev, e_tok, h_local):
    """x = [h_{t-1}, E(x_t), h^L_t] in the order the ODA page lists them."""
    return np.concatenate([np.asarray(h_prev, dtype=np.float64),
                           np.asarray(e_tok, dtype=np.float64),
                           np.asarray(h_local, dtype=np.float64)])


def gelu(a):
    """Exact GELU, a * Phi(a), with Phi the standard normal CDF."""
    a = np.asarray(a, dtype=np.float64)
    return a * 0.5 * (1.0 + erf(a / math.sqrt(2.0)))


def recall_score(x, W1, b1, w2, b2):
    """q_t for one input vector x = [h_{t-1}, E(x_t), h^L_t].

    W1: [hidden][in_dim], b1: [hidden], w2: [hidden], b2: scalar or [1].
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.asarray(W1, dtype=np.float64) @ x + np.asarray(b1, dtype=np.float64)
    u = gelu(a)
    return float(np.asarray(w2, dtype=np.float64) @ u + float(np.asarray(b2, dtype=np.float64).reshape(-1)[0]))


def gate(q_t, theta=0.0):
    """Recall decision: strictly greater than the threshold."""
    return bool(q_t > theta)
