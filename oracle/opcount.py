"""Multiply-accumulate cost model of generation with and without the cache -- TEST
INFRASTRUCTURE ONLY.

Follows gustavoai "La cache de claves y valores: cuanto cuesta cada token", section
"Lo que cuesta un token, con cache y sin ella", restated:

  * a matrix-vector product costs one multiplication per matrix entry; normalisation,
    softmax and activations are left out;
  * one row through the network costs c_row = L*(4*d_model^2 + 2*d_model*d_ff)
    + d_model*vocab (the q/k/v/output projections and the two MLP matrices per layer,
    then the output layer);
  * with the cache, the token at position t costs one row plus, in every layer, t dot
    products of d_k terms and the mix of t value rows over the h heads: 2*t*d_model;
  * without the cache, the token at position t re-runs all t rows: t times that.

The totals below are explicit loops over positions, so the closed forms printed on the
page (e.g. 8,921,088 vs 295,526,400 at T = 64 for the mini-GPT) are an independent check.
"""


def c_row(L, d_model, d_ff, vocab):
    return L * (4 * d_model * d_model + 2 * d_model * d_ff) + d_model * vocab


def cost_cached(t, L, d_model, d_ff, vocab):
    """MACs of the token at position t (1-based) when K/V of earlier positions are kept."""
    return c_row(L, d_model, d_ff, vocab) + L * 2 * t * d_model


def cost_uncached(t, L, d_model, d_ff, vocab):
    """MACs of the token at position t when the whole prefix is recomputed."""
    return t * cost_cached(t, L, d_model, d_ff, vocab)


def total_cached(T, **m):
    total = 0
    for t in range(1, T + 1):
        total += cost_cached(t, **m)
    return total


def total_uncached(T, **m):
    total = 0
    for t in range(1, T + 1):
        total += cost_uncached(t, **m)
    return total


def attention_equals_matrices_at(L, d_model, d_ff, vocab):
    """Smallest position t where the per-token attention MACs reach the matrix MACs."""
    t = 1
    while L * 2 * t * d_model < c_row(L, d_model, d_ff, vocab):
        t += 1
    return t


def score_bytes_per_step(n, elem_bytes, cached):
    """Score storage of one head for one generation step: the n x n matrix when the whole
    sequence is recomputed, a 1 x n row with the cache (neuralialabs chapter, one-head
    d = 64 comparison)."""
    return (n * elem_bytes) if cached else (n * n * elem_bytes)
