"""CPU oracle for tree verification of gated-delta-net layers -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may import this
module. It imports nothing from the HIP package.

Definition followed (DFlash-TfM summary page, "Rollback-free tree verification for GDN"): a
gated-delta-net layer keeps a matrix state S (d_k x d_v) per value head and updates it per token
as S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T. On a draft tree (nodes in
topological order, parent[i] in [-1, i-1]) every node continues its parent's state, and a
root-attached node continues the committed state S_0. Readings taken where the page is silent:

  * alpha_t = exp(g_t) with the log-decay g_t <= 0 given per node and value head; beta_t given;
  * the layer's output at node i is o_i = scale * S_i^T q_i (the state after the node's own update);
  * heads: H_k query/key heads and H_v value heads, value head h reading key head h // (H_v / H_k);
  * the committed state after acceptance is the state of the last accepted node (nothing else is
    written, so no rollback is needed).

This oracle is that recurrence written out, node by node, in fp64 -- not the chunked triangular
solve the GPU uses.
"""
from __future__ import annotations

import numpy as np


def _widen(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        a = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return a.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _check_parent(parent):
    B, T = parent.shape
    for b in range(B):
        for i in range(T):
            pa = int(parent[b, i])
            if pa < -1 or pa >= i:
                raise ValueError(f"parent[{b}][{i}] = {pa} is not in [-1, {i - 1}]")


def node_states(q, k, v, g, beta, parent, S0, b, h, dtype="bf16"):
    """Every node's state S_i (fp64 [T, d_k, d_v]) for sequence b, value head h."""
    T = parent.shape[1]
    Hk, Hv = k.shape[2], v.shape[2]
    hk = h // (Hv // Hk)
    K = _widen(k[b, :, hk], dtype)
    Vv = _widen(v[b, :, h], dtype)
    S0h = np.asarray(S0[b, h], np.float64)
    S = np.empty((T,) + S0h.shape)
    for i in range(T):
        pa = int(parent[b, i])
        prev = S0h if pa < 0 else S[pa]
        a = np.exp(float(g[b, i, h]))
        bt = float(beta[b, i, h])
        ki = K[i]
        # alpha (I - beta k k^T) S_prev, with (k k^T) S_prev taken as k (k^T S_prev)
        S[i] = a * (prev - bt * np.outer(ki, ki @ prev)) + bt * np.outer(ki, Vv[i])
    return S


def gdn_tree_verify(q, k, v, g, beta, parent, S0, scale, dtype="bf16"):
    """q, k: [B, T, H_k, d_k] (bf16 bits or fp32); v: [B, T, H_v, d_v]; g, beta: fp32
    [B, T, H_v]; parent int32 [B, T]; S0 fp32 [B, H_v, d_k, d_v]. Returns o fp64
    [B, T, H_v, d_v], o_i = scale * S_i^T q_i."""
    _check_parent(parent)
    B, T = parent.shape
    Hk, Hv = k.shape[2], v.shape[2]
    out = np.empty((B, T, Hv, v.shape[3]))
    for b in range(B):
        for h in range(Hv):
            S = node_states(q, k, v, g, beta, parent, S0, b, h, dtype)
            Q = _widen(q[b, :, h // (Hv // Hk)], dtype)
            out[b, :, h] = scale * np.einsum("tkv,tk->tv", S, Q)
    return out


def gdn_commit(q, k, v, g, beta, parent, S0, last, dtype="bf16"):
    """The committed states after acceptance: for every sequence b, the state of node last[b]
    (S0 unchanged where last[b] < 0). Returns fp64 [B, H_v, d_k, d_v]."""
    _check_parent(parent)
    B = parent.shape[0]
    Hv = v.shape[2]
    out = np.asarray(S0, np.float64).copy()
    for b in range(B):
        if last[b] < 0:
            continue
        for h in range(Hv):
            out[b, h] = node_states(q, k, v, g, beta, parent, S0, b, h, dtype)[last[b]]
    return out
