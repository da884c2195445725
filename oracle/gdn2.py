"""float64 oracle for the Gated DeltaNet-2 recurrence and its VJP (plain numpy,
sequential in time).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this module; the device library and
its Python binding never import it.

The recurrence is the direct graph of the burn_gdn source page
"src/chunk_wy/custom_backward.rs" (function ``forward_impl``).  Per batch
entry and head, with a state S of shape [latent, dense], S[-1] = the initial
state, and for t = 0 .. T-1 (vectors over latent: q, k, b = erase,
g = log_decay; over dense: v, w = write):

    a       = exp(g_t)                       decay, one factor per latent row
    D       = diag(a) S[t-1]                 decayed state
    e       = b_t * k_t                      erased key
    u       = w_t * v_t - D^T e              update (write minus erased read-out)
    S[t]    = D + k_t u^T                    rank-1 write
    o_t     = S[t]^T q_t / sqrt(latent)      context

returning the context [B, H, T, dense] and the final state S[T-1].  The chunk
size of the page's kernels does not change this result.

The VJP is the reverse sweep of that recurrence, as the page's generic
recompute backward (``backward_impl``) takes it, here over the whole saved
trajectory of states: given the context's cotangent do_t (and optionally the
final state's, zero on the page), with G the cotangent reaching S[t]

    G      += q_t do_t^T / sqrt(latent)
    d q_t   = S[t] do_t / sqrt(latent)
    d u     = G^T k_t,          d k_t  = G u + (D du_neg) * b_t   (du_neg = -d u)
    d w_t   = d u * v_t,        d v_t  = d u * w_t
    dD      = G + e du_neg^T
    d b_t   = (D du_neg) * k_t
    d g_t   = rowsum(dD * S[t-1]) * a
    G       = diag(a) dD                     (cotangent of S[t-1])

and the initial state's cotangent is the final G.

Arrays: query, key, erase, log_decay [B, H, T, L]; value, write [B, H, T, D];
initial_state, state [B, H, L, D]; context [B, H, T, D].
"""
from __future__ import annotations

import numpy as np

NAMES = ("query", "key", "value", "erase", "write", "log_decay", "initial_state")


def _f64(*arrays):
    return [np.asarray(x, dtype=np.float64) for x in arrays]


def _check(q, k, v, b, w, g, s0):
    B, H, T, L = q.shape
    D = v.shape[3]
    for name, x, shp in (("key", k, (B, H, T, L)), ("erase", b, (B, H, T, L)), ("log_decay", g, (B, H, T, L)),
                         ("value", v, (B, H, T, D)), ("write", w, (B, H, T, D)),
                         ("initial_state", s0, (B, H, L, D))):
        if x.shape != shp:
            raise ValueError(f"{name} must be {shp}, got {x.shape}")
    return B, H, T, L, D


def gdn2_states(query, key, value, erase, write, log_decay, initial_state):
    """(context, states) with states[:, :, t] = S[t-1] for t = 0 .. T (so
    states[:, :, 0] is the initial state and states[:, :, T] the final one)."""
    q, k, v, b, w, g, s0 = _f64(query, key, value, erase, write, log_decay, initial_state)
    B, H, T, L, D = _check(q, k, v, b, w, g, s0)
    scale = 1.0 / np.sqrt(L)
    states = np.empty((B, H, T + 1, L, D))
    ctx = np.empty((B, H, T, D))
    S = s0.copy()
    states[:, :, 0] = S
    for t in range(T):
        a = np.exp(g[:, :, t])                                   # [B, H, L]
        Dd = a[..., None] * S                                     # decayed state
        e = b[:, :, t] * k[:, :, t]                               # erased key
        u = w[:, :, t] * v[:, :, t] - np.einsum("bhld,bhl->bhd", Dd, e)
        S = Dd + k[:, :, t][..., None] * u[:, :, None, :]         # rank-1 write
        ctx[:, :, t] = scale * np.einsum("bhld,bhl->bhd", S, q[:, :, t])
        states[:, :, t + 1] = S
    return ctx, states


def gdn2_fwd(query, key, value, erase, write, log_decay, initial_state):
    """(context [B, H, T, D], final state [B, H, L, D])."""
    ctx, states = gdn2_states(query, key, value, erase, write, log_decay, initial_state)
    return ctx, states[:, :, -1].copy()


def gdn2_bwd(query, key, value, erase, write, log_decay, initial_state, d_context, d_state=None):
    """Cotangents of (query, key, value, erase, write, log_decay,
    initial_state) for the cotangent d_context of the context and, optionally,
    d_state of the final state (zero if None)."""
    q, k, v, b, w, g, s0, do = _f64(query, key, value, erase, write, log_decay, initial_state, d_context)
    B, H, T, L, D = _check(q, k, v, b, w, g, s0)
    if do.shape != (B, H, T, D):
        raise ValueError("d_context must have the context's shape")
    scale = 1.0 / np.sqrt(L)
    _, states = gdn2_states(q, k, v, b, w, g, s0)
    grads = {n: np.zeros_like(x) for n, x in zip(NAMES[:6], (q, k, v, b, w, g))}
    G = np.zeros((B, H, L, D)) if d_state is None else np.array(d_state, dtype=np.float64)
    for t in range(T - 1, -1, -1):
        S_prev, S_t = states[:, :, t], states[:, :, t + 1]
        a = np.exp(g[:, :, t])
        Dd = a[..., None] * S_prev
        e = b[:, :, t] * k[:, :, t]
        u = w[:, :, t] * v[:, :, t] - np.einsum("bhld,bhl->bhd", Dd, e)
        # read-out o_t = scale * S_t^T q_t
        G = G + scale * q[:, :, t][..., None] * do[:, :, t][:, :, None, :]
        grads["query"][:, :, t] = scale * np.einsum("bhld,bhd->bhl", S_t, do[:, :, t])
        # rank-1 write S_t = Dd + k u^T
        du = np.einsum("bhld,bhl->bhd", G, k[:, :, t])
        dk = np.einsum("bhld,bhd->bhl", G, u)
        # update u = w * v - Dd^T e
        grads["write"][:, :, t] = du * v[:, :, t]
        grads["value"][:, :, t] = du * w[:, :, t]
        dread = -du                                              # cotangent of Dd^T e
        dDd = G + e[..., None] * dread[:, :, None, :]
        de = np.einsum("bhld,bhd->bhl", Dd, dread)
        grads["erase"][:, :, t] = de * k[:, :, t]
        grads["key"][:, :, t] = dk + de * b[:, :, t]
        # decay Dd = diag(a) S_prev, a = exp(g)
        grads["log_decay"][:, :, t] = np.sum(dDd * S_prev, axis=-1) * a
        G = a[..., None] * dDd
    return (grads["query"], grads["key"], grads["value"], grads["erase"], grads["write"], grads["log_decay"], G)
