"""Pure-Python brute force of the attention definitions, for pinning the oracle.

Written independently of oracle/: plain nested loops over Python floats with
math.exp / math.log and math.fsum, no NumPy.  Only for tiny shapes.
"""
import math

NEG_INF = float("-inf")


def attend_row(qrow, keys, vals, padded, scale):
    """One query row against a list of key / value rows. Returns (out, lse)."""
    s = []
    for j, kr in enumerate(keys):
        if padded[j]:
            s.append(NEG_INF)
        else:
            s.append(scale * math.fsum(a * b for a, b in zip(qrow, kr)))
    m = max(s) if s else NEG_INF
    if m == NEG_INF:
        return [0.0] * len(vals[0]) if vals else [], NEG_INF
    e = [0.0 if x == NEG_INF else math.exp(x - m) for x in s]
    l = math.fsum(e)
    D = len(vals[0])
    out = [math.fsum(e[j] * vals[j][d] for j in range(len(vals))) / l for d in range(D)]
    return out, m + math.log(l)


def attention(q, k, v, mask, scale):
    """q [B][H][Tq][D] nested lists etc.; mask [B][Tk] (truthy = padded) or None."""
    B, H, Tq = len(q), len(q[0]), len(q[0][0])
    Tk = len(k[0][0])
    O = [[[None] * Tq for _ in range(H)] for _ in range(B)]
    L = [[[None] * Tq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        pad = [bool(mask[b][j]) if mask is not None else False for j in range(Tk)]
        for h in range(H):
            for i in range(Tq):
                O[b][h][i], L[b][h][i] = attend_row(q[b][h][i], k[b][h], v[b][h], pad, scale)
    return O, L


def merge(outs, lses):
    """Elementwise merge of n (out row, lse) pairs given as flat lists of rows."""
    n = len(outs)
    res_o, res_l = [], []
    for r in range(len(lses[0])):
        ls = [lses[i][r] for i in range(n)]
        M = max(ls)
        if M == NEG_INF:
            res_o.append([0.0] * len(outs[0][r]))
            res_l.append(NEG_INF)
            continue
        tot = math.fsum(math.exp(x - M) for x in ls)
        lse = M + math.log(tot)
        w = [math.exp(x - lse) for x in ls]
        res_o.append([math.fsum(w[i] * outs[i][r][d] for i in range(n)) for d in range(len(outs[0][r]))])
        res_l.append(lse)
    return res_o, res_l


def decode(q, kc, vc, lens, scale):
    """q [B][Hq][D] (the single token), caches [B][Hkv][T][D], lens [B]."""
    B, Hq = len(q), len(q[0])
    Hkv = len(kc[0])
    G = Hq // Hkv
    O = [[None] * Hq for _ in range(B)]
    L = [[None] * Hq for _ in range(B)]
    for b in range(B):
        n = int(lens[b])
        for h in range(Hq):
            g = h // G
            O[b][h], L[b][h] = attend_row(q[b][h], kc[b][g][:n], vc[b][g][:n], [False] * n, scale)
    return O, L
