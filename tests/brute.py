"""Pure-Python brute-force attention for tiny shapes (checks the C oracle).

Written independently of ``oracle/oracle.c``: masks are evaluated from
explicit per-token document ids, the soft cap uses ``math.tanh``, and every
sum is a plain Python loop.  Only for N <= ~16, d <= ~8.
"""
import math


def bf16_to_float(bits):
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def doc_ids_from_offsets(offsets, N):
    ids = [0] * N
    doc = -1
    starts = set(int(x) for x in offsets if int(x) < N)
    for i in range(N):
        if i in starts:
            doc += 1
        ids[i] = doc
    return ids


def attention(q, k, v, scale, causal=False, window=None, doc_offsets=None,
              softcap=None, alibi_slopes=None):
    """q [B][Hq][N][d], k/v [B][Hkv][N][d] nested lists of floats;
    alibi_slopes: per query head, the score loses slope * |i - j|.

    Returns O [B][Hq][N][d], LSE [B][Hq][N] as nested lists of floats."""
    B, Hq, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    group = Hq // Hkv
    if window is None:
        wl = wr = None
    elif isinstance(window, int):
        wl = wr = window
    else:
        wl, wr = window
    O = []
    L = []
    for b in range(B):
        ids = doc_ids_from_offsets(doc_offsets[b], N) if doc_offsets is not None else None
        Ob, Lb = [], []
        for h in range(Hq):
            hk = h // group
            Oh, Lh = [], []
            for i in range(N):
                scores = []
                for j in range(N):
                    ok = True
                    if causal and j > i:
                        ok = False
                    if wl is not None and not (i - wl <= j <= i + wr):
                        ok = False
                    if ids is not None and ids[i] != ids[j]:
                        ok = False
                    if not ok:
                        continue
                    dot = 0.0
                    for t in range(d):
                        dot += q[b][h][i][t] * k[b][hk][j][t]
                    s = dot * scale
                    if alibi_slopes is not None:
                        s -= alibi_slopes[h] * abs(i - j)
                    if softcap is not None:
                        s = softcap * math.tanh(s / softcap)
                    scores.append((j, s))
                if not scores:
                    Oh.append([0.0] * d)
                    Lh.append(-math.inf)
                    continue
                mx = max(s for _, s in scores)
                den = 0.0
                for _, s in scores:
                    den += math.exp(s - mx)
                out = [0.0] * d
                for j, s in scores:
                    w = math.exp(s - mx) / den
                    for t in range(d):
                        out[t] += w * v[b][hk][j][t]
                Oh.append(out)
                Lh.append(mx + math.log(den))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return O, L


def attention_varlen(q, k, v, cu_q, cu_k, scale, causal=False, window=None, softcap=None):
    """Packed variable-length attention by loops.  q [tq][Hq][d], k/v
    [tk][Hkv][d] nested lists of floats; cu_q, cu_k cumulative lengths.
    Query i of a sequence (local index) sees local key j when
    j <= i + Lk - Lq (causal) and |j - (i + Lk - Lq)| is inside the window.

    Returns O [tq][Hq][d], LSE [Hq][tq]."""
    tq, Hq, d = len(q), len(q[0]) if q else 0, len(q[0][0]) if q else 0
    Hkv = len(k[0]) if k else 1
    group = Hq // Hkv if Hkv else 1
    if window is None:
        wl = wr = None
    elif isinstance(window, int):
        wl = wr = window
    else:
        wl, wr = window
    O = [[None] * Hq for _ in range(tq)]
    L = [[None] * tq for _ in range(Hq)]
    for s in range(len(cu_q) - 1):
        lq, lk = cu_q[s + 1] - cu_q[s], cu_k[s + 1] - cu_k[s]
        for il in range(lq):
            i = cu_q[s] + il
            shift = il + lk - lq
            for h in range(Hq):
                hk = h // group
                scores = []
                for jl in range(lk):
                    if causal and jl > shift:
                        continue
                    if wl is not None and not (shift - wl <= jl <= shift + wr):
                        continue
                    j = cu_k[s] + jl
                    dot = 0.0
                    for t in range(d):
                        dot += q[i][h][t] * k[j][hk][t]
                    sc = dot * scale
                    if softcap is not None:
                        sc = softcap * math.tanh(sc / softcap)
                    scores.append((j, sc))
                if not scores:
                    O[i][h] = [0.0] * d
                    L[h][i] = -math.inf
                    continue
                mx = max(sc for _, sc in scores)
                den = 0.0
                for _, sc in scores:
                    den += math.exp(sc - mx)
                out = [0.0] * d
                for j, sc in scores:
                    w = math.exp(sc - mx) / den
                    for t in range(d):
                        out[t] += w * v[j][hk][t]
                O[i][h] = out
                L[h][i] = mx + math.log(den)
    return O, L
