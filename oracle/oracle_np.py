"""NumPy float64 oracle for the fused attention forward and its gradients.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke entry point
and the benchmark's CPU-baseline leg, never by the HIP library or its binding.
It is written independently of ``fa_oracle.c`` (the C oracle) so the two can
cross-check each other; they share no code.

Definition followed (plain, materialised, float64):
  * "[CS336] Assignment 2: Systems", section "FlashAttention V2 / High level":
    S = Q K^T scaled, P = row-softmax(S), O = P V, and the per-row logsumexp
    L_i = log sum_j exp(S_ij).
  * "Understanding Triton Tutorials Part 2", section "Fused Attention 2": the
    causal mask is the lower triangle (key j visible to query i iff j <= i)
    and the softmax is taken after subtracting the row maximum.
Readings where the pages are silent: top-left causal alignment when
seq_q != seq_k; keys j >= seq_k do not exist; natural-log lse; the scale
multiplies the exact dot product; P is not rounded before P V.
"""
import numpy as np


def attention_forward(q, k, v, sm_scale, causal, row_block=256):
    """q: [B, H, Sq, D], k/v: [B, H, Sk, D] float64 arrays.

    Returns (o [B, H, Sq, D], lse [B, H, Sq]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if Sk < 1:
        raise ValueError("softmax over an empty key set is undefined")
    o = np.empty((B, H, Sq, D), dtype=np.float64)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    key_idx = np.arange(Sk)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, row_block):
                rows = np.arange(r0, min(Sq, r0 + row_block))
                scores = (q[b, h, rows] @ k[b, h].T) * sm_scale
                if causal:
                    hidden = key_idx[None, :] > rows[:, None]
                    scores = np.where(hidden, -np.inf, scores)
                row_max = scores.max(axis=1, keepdims=True)
                unnorm = np.exp(scores - row_max)
                denom = unnorm.sum(axis=1, keepdims=True)
                o[b, h, rows] = (unnorm / denom) @ v[b, h]
                lse[b, h, rows] = row_max[:, 0] + np.log(denom[:, 0])
    return o, lse


def attention_forward_tiled(q, k, v, sm_scale, causal, block_m, block_n, lazy_threshold=0.0):
    """The tiled online-softmax recurrence, in float64 -- the algorithm of
    "[CS336] Assignment 2: Systems", section "FlashAttention V2: Forward Pass"
    and of the inner loop of "Understanding Triton Tutorials Part 2",
    section "Fused Attention 2", written out block by block: for each block of
    ``block_m`` query rows, walk the key blocks of ``block_n`` keys keeping a
    running maximum m, a running sum l and an unnormalised output O~; for a key
    block with scores S (masked entries -inf)
        m_new = max(m, rowmax S),  P = exp(S - m_new),
        l = exp(m - m_new) l + rowsum P,  O~ = exp(m - m_new) O~ + P V,
    then O = O~ / l and lse = m + log l.

    ``lazy_threshold`` > 0 models the reading that m is only refreshed when the
    block maximum exceeds it by more than the threshold (natural-log units);
    any reference maximum gives the same O and lse in exact arithmetic.

    Not used to produce expected values: it is pinned against the plain
    definition (``attention_forward``) in the tests.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    o = np.empty((B, H, Sq, D), dtype=np.float64)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, block_m):
                rows = np.arange(r0, min(Sq, r0 + block_m))
                m = np.full(rows.size, -np.inf)
                l = np.zeros(rows.size)
                acc = np.zeros((rows.size, D))
                for c0 in range(0, Sk, block_n):
                    cols = np.arange(c0, min(Sk, c0 + block_n))
                    s = (q[b, h, rows] @ k[b, h, cols].T) * sm_scale
                    if causal:
                        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
                    m_blk = s.max(axis=1)
                    m_new = np.maximum(m, m_blk)
                    if lazy_threshold > 0:
                        m_new = np.where(m_blk > m + lazy_threshold, m_new, m)
                    # rows with nothing visible so far keep m = -inf and add nothing
                    ref = np.where(np.isfinite(m_new), m_new, 0.0)
                    p = np.exp(s - ref[:, None])
                    alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, h, cols]
                    m = m_new
                o[b, h, rows] = acc / l[:, None]
                lse[b, h, rows] = m + np.log(l)
    return o, lse


def attention_backward_tiled(q, k, v, dout, sm_scale, causal, block_m, block_n):
    """The two-phase tiled backward, in float64 -- the blocked form of
    "[CS336] Assignment 2: Systems", section "FlashAttention V2: Backward
    Pass", split as that page's Triton version splits it: with O and L from
    the plain forward (``attention_forward``) and D = rowsum(dO o O),
      phase 1, per block of ``block_m`` queries, over the key blocks:
        P = exp(S - L) (masked entries 0), dP = dO V^T, dS = P o (dP - D),
        dQ += scale dS K;
      phase 2, per block of ``block_n`` keys, over the query blocks:
        the same P and dS, dV += P^T dO, dK += scale dS^T Q.
    Each phase recomputes P.  Not used to produce expected values: it is
    pinned against ``attention_backward`` in the tests.  Returns (dq, dk, dv).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    o, lse = attention_forward(q, k, v, sm_scale, causal)
    delta = np.sum(dout * o, axis=-1)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)

    def blocks(b, h, rows, cols):
        s = (q[b, h, rows] @ k[b, h, cols].T) * sm_scale
        p = np.exp(s - lse[b, h, rows][:, None])
        if causal:
            p = np.where(cols[None, :] > rows[:, None], 0.0, p)
        dp = dout[b, h, rows] @ v[b, h, cols].T
        ds = p * (dp - delta[b, h, rows][:, None])
        return p, ds

    for b in range(B):
        for h in range(H):
            for r0 in range(0, Sq, block_m):  # phase 1: dQ
                rows = np.arange(r0, min(Sq, r0 + block_m))
                for c0 in range(0, Sk, block_n):
                    cols = np.arange(c0, min(Sk, c0 + block_n))
                    _, ds = blocks(b, h, rows, cols)
                    dq[b, h, rows] += sm_scale * (ds @ k[b, h, cols])
            for c0 in range(0, Sk, block_n):  # phase 2: dK, dV
                cols = np.arange(c0, min(Sk, c0 + block_n))
                for r0 in range(0, Sq, block_m):
                    rows = np.arange(r0, min(Sq, r0 + block_m))
                    p, ds = blocks(b, h, rows, cols)
                    dv[b, h, cols] += p.T @ dout[b, h, rows]
                    dk[b, h, cols] += sm_scale * (ds.T @ q[b, h, rows])
    return dq, dk, dv


def attention_backward(q, k, v, dout, sm_scale, causal):
    """Gradients dQ, dK, dV of O = attention(q, k, v) for upstream dout.

    Materialised per (batch, head), float64.  Follows "[CS336] Assignment 2:
    Systems", section "FlashAttention V2": dV = P^T dO, dP = dO V^T,
    dS = P o (dP - rowsum(dO o O)), dQ = scale dS K, dK = scale dS^T Q, with
    P the row softmax of the scaled, masked scores.  Written apart from
    fa_oracle_bwd.c.  Returns (dq, dk, dv).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    visible = np.ones((Sq, Sk), dtype=bool)
    if causal:
        visible = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            s = sm_scale * (q[b, h] @ k[b, h].T)
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            o = p @ v[b, h]
            dv[b, h] = p.T @ dout[b, h]
            dp = dout[b, h] @ v[b, h].T
            ds = p * (dp - np.sum(dout[b, h] * o, axis=1, keepdims=True))
            dq[b, h] = sm_scale * (ds @ k[b, h])
            dk[b, h] = sm_scale * (ds.T @ q[b, h])
    return dq, dk, dv
