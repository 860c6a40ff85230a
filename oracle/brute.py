"""Independent brute force for tiny shapes -- TEST INFRASTRUCTURE ONLY.

Pure Python lists, math.fsum (exactly rounded sums) and math.exp.  It shares nothing with
kvp_oracle.c: it is a second, differently ordered evaluation of the same definitions, used
to pin the C oracle on small inputs (B <= 2, heads <= 4, n <= 9, d in {4, 8, 64}).

Definitions followed:
  * attention row -- the TraditionalAttention module of the chatgpz.de "Aufmerksamkeit"
    linear-attention post: softmax(q K^T / sqrt(d)) V;
  * decode attends over every cached position including the one just appended
    (gustavoai "La cache de claves y valores", four-step token recipe);
  * GQA head map h -> h // (Hq // Hkv) (xformers demo, section 5, BMGHK layout);
  * packed varlen prefill, block-diagonal (optionally causal) mask (xformers demo,
    section 4);
  * several new rows per request against its cache, each row over the positions up to its
    own (draft verification as one pass over gamma positions, "Tornar a inferencia
    barata" chapter, speculative-decoding section).
"""
import math


def attention_row(q, K, V, scale):
    """q: list[d]; K, V: list[n][d] -> (out list[d], p list[n])."""
    s = [scale * math.fsum(qc * kc for qc, kc in zip(q, krow)) for krow in K]
    # softmax: the exponentials are taken against the largest score, then normalised
    top = max(s)
    e = [math.exp(x - top) for x in s]
    z = math.fsum(e)
    p = [x / z for x in e]
    d = len(V[0])
    out = [math.fsum(p[j] * V[j][c] for j in range(len(V))) for c in range(d)]
    return out, p


def decode_gqa(q, K, V, ctx, scale):
    """q[B][Hq][d], K/V[B][Hkv][Lmax][d], ctx[B] -> out[B][Hq][d]."""
    B, Hq = len(q), len(q[0])
    Hkv = len(K[0])
    grp = Hq // Hkv
    out = []
    for b in range(B):
        rows = []
        for h in range(Hq):
            g = h // grp
            o, _ = attention_row(q[b][h], K[b][g][:ctx[b]], V[b][g][:ctx[b]], scale)
            rows.append(o)
        out.append(rows)
    return out


def varlen_prefill(q, k, v, cu, causal, scale):
    """q[T][Hq][d], k/v[T][Hkv][d], cu[nseg+1] -> out[T][Hq][d]."""
    T, Hq = len(q), len(q[0])
    Hkv = len(k[0])
    grp = Hq // Hkv
    out = [None] * T
    for s in range(len(cu) - 1):
        a, e = cu[s], cu[s + 1]
        for i in range(a, e):
            rows = []
            for h in range(Hq):
                g = h // grp
                last = i + 1 if causal else e
                Ks = [k[j][g] for j in range(a, last)]
                Vs = [v[j][g] for j in range(a, last)]
                o, _ = attention_row(q[i][h], Ks, Vs, scale)
                rows.append(o)
            out[i] = rows
    return out


def chunk_attention(q, K, V, ctx, cu, scale):
    """Several new rows per request against its cache: q[T][Hq][d] with request b's rows
    cu[b] .. cu[b+1]-1, K/V[B][Hkv][Lmax][d], ctx[B].  The m rows of request b are its
    last m positions; row i attends to positions 0 .. ctx[b] - m + i (the draft-verification
    pass of the "Tornar a inferencia barata" chapter, one forward pass over gamma positions)."""
    B, Hq = len(ctx), len(q[0])
    Hkv = len(K[0])
    grp = Hq // Hkv
    out = [None] * len(q)
    for b in range(B):
        m = cu[b + 1] - cu[b]
        for i in range(m):
            pos = ctx[b] - m + i  # this row's own position
            rows = []
            for h in range(Hq):
                g = h // grp
                o, _ = attention_row(q[cu[b] + i][h], K[b][g][:pos + 1], V[b][g][:pos + 1], scale)
                rows.append(o)
            out[cu[b] + i] = rows
    return out
