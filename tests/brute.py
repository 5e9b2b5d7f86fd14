"""Brute-force references written with explicit Python loops, used only to pin the oracle.

Nothing here imports the oracle or the HIP path. RoPE is written in its complex-number form
(x_i + i*x_{i+d/2}) * exp(i * p * theta_i), attention with per-head, per-token loops and
math.exp, selection with Python's sorted() on (-score, index) keys.
"""

import cmath
import math


def theta(d, base):
    return [base ** (-(2.0 * i) / d) for i in range(d // 2)]


def rope_complex(x, p, base):
    d = len(x)
    half = d // 2
    th = theta(d, base)
    out = [0.0] * d
    for i in range(half):
        z = complex(x[i], x[i + half]) * cmath.exp(1j * p * th[i])
        out[i] = z.real
        out[i + half] = z.imag
    return out


def kv_of(h, H_q, H_kv):
    return h * H_kv // H_q


def grp_of(g, H_kv, G):
    return g * G // H_kv


def dense_rope_attention(q, K, V, positions, T, base, H_q, H_kv, d):
    """o_h = sum_t softmax_t(RoPE(q_h, T-1) . RoPE(K[t, kv(h)], t) / sqrt(d)) V[t, kv(h)]
    over the given positions. q: [H_q][d]; K, V: [T][H_kv*d] pre-RoPE rows (nested lists)."""
    out = []
    for h in range(H_q):
        g = kv_of(h, H_q, H_kv)
        qr = rope_complex(list(q[h]), T - 1, base)
        logits = []
        for t in positions:
            kr = rope_complex(list(K[t][g * d:(g + 1) * d]), t, base)
            logits.append(sum(qr[c] * kr[c] for c in range(d)) / math.sqrt(d))
        m = max(logits)
        e = [math.exp(v - m) for v in logits]
        z = sum(e)
        o = [0.0] * d
        for j, t in enumerate(positions):
            for c in range(d):
                o[c] += e[j] / z * V[t][g * d + c]
        out.append(o)
    return out


def ropefree_group_scores(q, K, T_c, H_q, H_kv, G, d):
    """S[s][t] = sum over heads h with grp(kv(h)) = s of q_h . K[t, kv(h)] (no RoPE)."""
    S = [[0.0] * T_c for _ in range(G)]
    for h in range(H_q):
        g = kv_of(h, H_q, H_kv)
        s = grp_of(g, H_kv, G)
        for t in range(T_c):
            S[s][t] += sum(q[h][c] * K[t][g * d + c] for c in range(d))
    return S


def select(scores, T, k, w):
    T_c = max(0, T - w)
    kp = min(k, T_c)
    order = sorted(range(T_c), key=lambda t: (-scores[t], t))
    return sorted(order[:kp]) + list(range(T_c, T))


def causal_importance(Qobs, K, T):
    """I[t] = sum_i softmax over t' <= T-w+i of Qobs[i] . K[t'] / sqrt(d)."""
    w = len(Qobs)
    d = len(Qobs[0])
    I = [0.0] * T
    for i in range(w):
        p = T - w + i
        logits = [sum(Qobs[i][c] * K[t][c] for c in range(d)) / math.sqrt(d) for t in range(p + 1)]
        m = max(logits)
        e = [math.exp(v - m) for v in logits]
        z = sum(e)
        for t in range(p + 1):
            I[t] += e[t] / z
    return I


def masked_attention(q, K, V, keep):
    """softmax over the kept positions only (the others masked to -inf) of q . K / sqrt(d), times V."""
    d = len(q)
    logits = []
    for t in range(len(K)):
        logits.append(sum(q[c] * K[t][c] for c in range(d)) / math.sqrt(d) if t in keep else -math.inf)
    m = max(logits)
    e = [math.exp(v - m) if v != -math.inf else 0.0 for v in logits]
    z = sum(e)
    return [sum(e[t] / z * V[t][c] for t in range(len(K))) for c in range(d)]
