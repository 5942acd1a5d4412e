"""Pure-Python brute force (math.exp / math.fsum, no NumPy) used only to pin
the oracle.  Independent of oracle/: different code, different arithmetic."""
import math


def brute_attention(q, k, v, causal, window=None):
    """q: [T][h_q][d], k, v: [S][h_kv][d] nested lists.  Returns [T][h_q][d].
    window W (causal only): query i sees keys i - W < j <= i."""
    T, h_q, d = len(q), len(q[0]), len(q[0][0])
    S, h_kv = len(k), len(k[0])
    g = h_q // h_kv
    scale = 1.0 / math.sqrt(d)
    out = []
    for i in range(T):
        row = []
        for h in range(h_q):
            kv = h // g
            js = [j for j in range(S) if (not causal or j <= i) and (window is None or i - j < window)]
            sc = [scale * math.fsum(q[i][h][t] * k[j][kv][t] for t in range(d)) for j in js]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            den = math.fsum(w)
            row.append([math.fsum(w[n] * v[js[n]][kv][t] for n in range(len(js))) / den
                        for t in range(d)])
        out.append(row)
    return out


def brute_triplet(qrow, krows, vrows, admissible, scale):
    """(m, l, O) of one query row over the admissible keys, by hand."""
    sc = [scale * math.fsum(a * b for a, b in zip(qrow, kr)) for kr, ok in zip(krows, admissible) if ok]
    vs = [vr for vr, ok in zip(vrows, admissible) if ok]
    if not sc:
        return -math.inf, 0.0, [0.0] * len(qrow)
    m = max(sc)
    w = [math.exp(s - m) for s in sc]
    return m, math.fsum(w), [math.fsum(w[n] * vs[n][t] for n in range(len(vs))) for t in range(len(vrows[0]))]
