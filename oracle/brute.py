"""Brute-force twin of the block-sparse pass for tiny inputs (N <= 512), in pure Python.

TEST INFRASTRUCTURE ONLY (see oracle/solattn.py).  It re-derives the pass along
a different route from the block oracle, straight from the word statements on
the pages (the ComfyUI BlockSparseAttention node docs' input tables and the
star7 README's "Sol" and "SLA" sections):
  * block means and dot products by explicit loops with math.fsum;
  * row mean and population deviation from the statistics module;
  * top-k choices by Python's sorted() on (-score, index) keys;
  * the attention as a full N x N table: every (query row r, key token t) pair
    gets one weight and one value -- exactly (exp(c q_r.k_t), v_t) when t is in
    a kept block or an extra token, else the centroid pair
    (exp(c q_r.k̄_b(t)), v̄_b(t)) for sol, or nothing for sla -- and
    out_r = sum_t w u / sum_t w, with no grouping into blocks and no
    multiplicities.
"""
import math
import statistics


def _dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def _mean_rows(rows):
    n = len(rows)
    return [math.fsum(r[e] for r in rows) / n for e in range(len(rows[0]))]


def brute_head(mode, q, k, v, *, block_q, block_k, tau=1.3, keep_percent=10.0, sink_range=0,
               extra_tokens=0, dense_rows=(0, 0)):
    """q, k, v: lists (or arrays) [N][d].  Returns (out [N][d], kept sets, extra sets)."""
    q = [[float(x) for x in row] for row in q]
    k = [[float(x) for x in row] for row in k]
    v = [[float(x) for x in row] for row in v]
    N, d = len(q), len(q[0])
    c = 1.0 / math.sqrt(d)
    qblk = [list(range(lo, min(lo + block_q, N))) for lo in range(0, N, block_q)]
    kblk = [list(range(lo, min(lo + block_k, N))) for lo in range(0, N, block_k)]
    M = len(kblk)
    qbar = [_mean_rows([q[t] for t in b]) for b in qblk]
    kbar = [_mean_rows([k[t] for t in b]) for b in kblk]
    vbar = [_mean_rows([v[t] for t in b]) for b in kblk]
    block_of = {t: j for j, b in enumerate(kblk) for t in b}

    kept_sets, extra_sets = [], []
    for i, rows in enumerate(qblk):
        if all(dense_rows[0] <= r < dense_rows[1] for r in rows):
            kept_sets.append(set(range(M)))
            extra_sets.append(set())
            continue
        s = [c * _dot(qbar[i], kbar[j]) for j in range(M)]
        forced = {j for j in range(M)
                  if any(t < sink_range for t in kblk[j]) or set(kblk[j]) & set(rows)}
        if mode == "sol":
            if tau == -math.inf:
                kept = set(range(M))
            else:
                mu = statistics.fmean(s)
                sd = statistics.pstdev(s, mu)
                theta = mu + tau * sd if sd > 0 else mu
                kept = forced | {j for j in range(M) if s[j] > theta}
        else:
            free = sorted((j for j in range(M) if j not in forced), key=lambda j: (-s[j], j))
            kcount = min(len(free), int(math.ceil(float(keep_percent) * M / 100.0)))
            kept = forced | set(free[:kcount])
        cand = [t for t in range(N) if block_of[t] not in kept]
        ranked = sorted(cand, key=lambda t: (-_dot(qbar[i], k[t]), t))
        extra = set(ranked[:max(0, extra_tokens)])
        kept_sets.append(kept)
        extra_sets.append(extra)

    out = []
    for i, rows in enumerate(qblk):
        for r in rows:
            terms = []                      # (logit, value vector) per key token
            for t in range(N):
                if dense_rows[0] <= r < dense_rows[1]:
                    terms.append((c * _dot(q[r], k[t]), v[t]))
                elif block_of[t] in kept_sets[i] or t in extra_sets[i]:
                    terms.append((c * _dot(q[r], k[t]), v[t]))
                elif mode == "sol":
                    j = block_of[t]
                    terms.append((c * _dot(q[r], kbar[j]), vbar[j]))
            L = max(lg for lg, _ in terms)
            w = [math.exp(lg - L) for lg, _ in terms]
            den = math.fsum(w)
            out.append([math.fsum(wi * u[e] for wi, (_, u) in zip(w, terms)) / den
                        for e in range(d)])
    return out, kept_sets, extra_sets
