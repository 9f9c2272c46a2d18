"""fp64 gradients of the HiLS attention forward -- TEST INFRASTRUCTURE.

Only ``tests/`` and ``bench.py``'s CPU leg may use this module; it shares no
code with the GPU library.  Plain numpy, one query row at a time, in the
order of the forward definition (hyper.ai HiLS summary, section 方法: the
landmark distribution, compressed key and entropy bias; the surrogate chunk
score; the partition estimate and the hierarchical factorisation of the
attention weight), with the selection held fixed (top-K is a discrete
choice; gradients flow through the selected chunks' scores).

For a row i of query head h (landmark head l, kv head g) with selection I:
  forward   a_j = s_j = scale q.k_j (window keys), a_j = s_j + s^_c - lse_c
            (keys of selected chunk c), L = LSE_j a_j, o = sum_j e^{a_j - L} v_j
            -- the fused output written as one softmax (bias form);
  backward  with loss dO.o + dL.L and P_j = e^{a_j - L}:
            dA_j = P_j (dO.v_j - dO.o + dL)
            window key:          ds_j = dA_j
            key of chunk c:      ds_j = w_c p_cj (dO.v_j - dO.o_c),  w_c = e^{s^_c - L}
            chunk score:         ds^_c = sum_{j in c} dA_j = w_c (dO.o_c - dO.o + dL)
            dv_j += P_j dO;  dq += scale sum_j ds_j k_j + scale sum_c ds^_c k'_c
            dk_j += scale ds_j q;  dk'_c += scale ds^_c q;  db'_c += ds^_c
  summary   (per chunk c and landmark head l, a_j = scale q'.k_j, p = softmax a,
            k' = sum p_j k_j, b' = LSE(a) - p.a):
            da_j = p_j (dk'.(k_j - k')) - db' p_j (a_j - p.a)
            dq' = scale sum_j da_j k_j;  dk_j += p_j dk' + scale da_j q'
The scoring query is the raw q (no Q-Cal).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import logsumexp


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def backward(cfg: dict, q, k, v, q_lm, sel_idx, dout, dlse=None, landmark: str = "chunk", rows=None):
    """Gradients of sum(dout * out) + sum(dlse * lse) for a prefill with the
    given selection.

    q [B,H_q,N,d]; k, v [B,H_kv,N,d]; q_lm [B,H_lm,C,d] ([H_lm,d] for
    "shared": one query per landmark head for every chunk; None for "mean");
    sel_idx [B,H_kv,N,K] (ascending, -1 padded); dout [B,H_q,N,d];
    dlse [B,H_q,N] or None.  Returns dict(dq, dk, dv, dq_lm, out, lse,
    sel_score, dsel) in float64 (dq_lm None for "mean", [H_lm,d] for
    "shared"; dsel = ds^ per selected slot [B,H_q,N,K], 0 on padding).
    rows: optional query positions to visit (default all).  The loss is
    linear in dout and dlse, so a row whose dout and dlse vanish contributes
    nothing to any gradient: with dout = dlse = 0 outside ``rows`` the
    gradients are exactly those of the full loop (out, lse and sel_score are
    then filled for the visited rows only).  Then, too, only the chunks that
    a visited row selected get their summaries and summary backward: every
    other chunk's dk' and db' are zero, so its summary backward adds nothing.
    """
    B, H_q, N, d = np.shape(q)
    H_kv = np.shape(k)[1]
    H_lm = int(cfg.get("H_lm", H_q))
    S, W, K = int(cfg["S"]), int(cfg["W"]), int(cfg["K"])
    scale = float(cfg.get("scale") or 1.0 / math.sqrt(d))
    G = H_q // H_kv
    C = N // S
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    sel = np.asarray(sel_idx.detach().cpu().numpy() if hasattr(sel_idx, "detach") else sel_idx, dtype=np.int64)
    dl = np.zeros((B, H_q, N)) if dlse is None else _f64(dlse)
    if landmark == "chunk":
        ql = _f64(q_lm)
    elif landmark == "shared":
        ql = np.broadcast_to(_f64(q_lm)[None, :, None, :], (B, H_lm, C, d)).copy()
    else:
        assert landmark == "mean", landmark
        ql = np.zeros((B, H_lm, C, d))

    def kv_of_lm(l):
        return l * H_kv // H_lm

    def lm_of(h):
        return h * H_lm // H_q

    # chunks whose summaries enter the visited rows (all of them without rows)
    used = np.ones((B, H_kv, C), bool)
    if rows is not None:
        used[:] = False
        for b in range(B):
            for g in range(H_kv):
                for i in rows:
                    cs = sel[b, g, i]
                    used[b, g, cs[cs >= 0]] = True

    # summaries (forward), kept with their softmax for the summary backward
    ksum = np.zeros((B, H_lm, C, d))
    bsum = np.zeros((B, H_lm, C))
    pl = np.zeros((B, H_lm, C, S))
    al = np.zeros((B, H_lm, C, S))
    for b in range(B):
        for l in range(H_lm):
            g = kv_of_lm(l)
            for c in range(C):
                if not used[b, g, c]:
                    continue
                kc = k[b, g, c * S:(c + 1) * S]
                a = scale * kc @ ql[b, l, c]
                p = np.exp(a - logsumexp(a))
                ksum[b, l, c] = p @ kc
                bsum[b, l, c] = logsumexp(a) - p @ a
                pl[b, l, c], al[b, l, c] = p, a

    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dks = np.zeros_like(ksum)
    dbs = np.zeros_like(bsum)
    out = np.zeros((B, H_q, N, d))
    lse = np.zeros((B, H_q, N))
    sel_score = np.full((B, H_q, N, K), -np.inf)
    dsel = np.zeros((B, H_q, N, K))
    for b in range(B):
        for h in range(H_q):
            g, l = h // G, lm_of(h)
            for i in (range(N) if rows is None else rows):
                qi, doi = q[b, h, i], do[b, h, i]
                w0 = max(0, (i // S) * S - W)
                # forward: the effective logits of every attended key
                keys, logits, chunk_of = [], [], []
                wj = np.arange(w0, i + 1)
                keys.append(wj)
                logits.append(scale * k[b, g, wj] @ qi)
                chunk_of.append(np.full(len(wj), -1))
                slots = [(kk, int(c)) for kk, c in enumerate(sel[b, g, i]) if c >= 0]
                shat = {}
                for kk, c in slots:
                    cj = np.arange(c * S, c * S + S)
                    s = scale * k[b, g, cj] @ qi
                    shat[c] = scale * qi @ ksum[b, l, c] + bsum[b, l, c]
                    sel_score[b, h, i, kk] = shat[c]
                    keys.append(cj)
                    logits.append(s + shat[c] - logsumexp(s))
                    chunk_of.append(np.full(S, c))
                keys, a, chunk_of = np.concatenate(keys), np.concatenate(logits), np.concatenate(chunk_of)
                L = logsumexp(a)
                P = np.exp(a - L)
                o = P @ v[b, g, keys]
                out[b, h, i], lse[b, h, i] = o, L
                # backward
                dov = v[b, g, keys] @ doi
                dA = P * (dov - doi @ o + dl[b, h, i])
                ds = dA.copy()
                for kk, c in slots:
                    m = chunk_of == c
                    pc = P[m] / P[m].sum()
                    oc = pc @ v[b, g, keys[m]]
                    wc = P[m].sum()  # = e^{s^_c - L}
                    ds[m] = wc * pc * (dov[m] - doi @ oc)
                    dsh = dA[m].sum()
                    dsel[b, h, i, kk] = dsh
                    dq[b, h, i] += scale * dsh * ksum[b, l, c]
                    dks[b, l, c] += scale * dsh * qi
                    dbs[b, l, c] += dsh
                dv[b, g, keys] += np.outer(P, doi)
                dq[b, h, i] += scale * ds @ k[b, g, keys]
                dk[b, g, keys] += scale * np.outer(ds, qi)
    # summary backward
    dql = np.zeros_like(ql)
    for b in range(B):
        for l in range(H_lm):
            g = kv_of_lm(l)
            for c in range(C):
                if not used[b, g, c]:
                    continue
                kc = k[b, g, c * S:(c + 1) * S]
                p, a = pl[b, l, c], al[b, l, c]
                da = p * ((kc - ksum[b, l, c]) @ dks[b, l, c]) - dbs[b, l, c] * p * (a - p @ a)
                dql[b, l, c] = scale * da @ kc
                dk[b, g, c * S:(c + 1) * S] += np.outer(p, dks[b, l, c]) + scale * np.outer(da, ql[b, l, c])
    # the shared query's gradient collects every chunk's
    dq_lm = {"chunk": dql, "shared": dql.sum(axis=(0, 2)), "mean": None}[landmark]
    return dict(dq=dq, dk=dk, dv=dv, dq_lm=dq_lm, out=out, lse=lse, sel_score=sel_score, dsel=dsel)
