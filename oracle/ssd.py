"""Plain fp64 CPU oracle of the batched lossless verify-and-resample step.

Test infrastructure only: imported by tests/, the smoke check and the CPU
baseline of the benchmark, never by the product path.  It shares no code,
constants table or helper with the GPU library; both follow the same written
specification.

Sources (web pages on Speculative Speculative Decoding, SSD, and its Saguaro
algorithm), cited by title and section:

[SSD-A] "全球最強推理引擎還快2倍，斯坦福、普林斯頓破解大模型串行魔咒"
        (a repost of a 機器之心 article), section "SSD 如何實現草擬與驗證并行？".
[SSD-B] "超越传统SD：SSD框架全异步解码实现4.7倍平均加速", sections
        "投机解码的瓶颈与 SSD 的核心机制" and "Saguaro 算法：解决异步推测的三大挑战"
        with its parts "1. 验证结果预测与缓存拓扑优化", "2. 操纵残差分布" and
        "3. 大 Batch 下的退避策略".

Every formula on [SSD-B] was lost when the page was extracted, so the exact
forms below are readings; each reading is named where it is used.  The
acceptance rule and the residual are the textbook speculative-sampling rule
(Leviathan, Kalman, Matias, ICML 2023; Chen et al. 2023), which [SSD-A]
describes in words (the target decides how many drafted tokens to accept and
then samples one extra bonus token, and the output follows the target's
distribution).

Parity unpinned: the cost model of backoff() is a reading the pages do not
fix (they give no formula for the back-off decision); its algebra is pinned
(ties, the closed-form critical batch, limiting cases), its content is not.

Arrays: logits z are fp64 with the vocabulary last.  A row has V entries;
-inf marks a token of zero weight.  Temperatures that are not > 0 select the
greedy (argmax) path.
"""
import math

import numpy as np

from . import philox as ph

BLK = 2048  # vocabulary block of the two-level sampler


# --------------------------------------------------------------------------
# decoding of the stored logits
# --------------------------------------------------------------------------
def decode(raw, dtype):
    """Exact decode of stored logits to fp64.

    bf16 and fp16 are given as their 16-bit patterns (any 16-bit integer
    dtype) or, for fp16, as numpy float16; fp32 as float32.
    """
    raw = np.asarray(raw)
    if dtype == "bf16":
        bits = raw.view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f16":
        if raw.dtype != np.float16:
            raw = raw.view(np.float16)
        return raw.astype(np.float64)
    if dtype == "f32":
        return raw.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def is_greedy(T):
    return not (T > 0)


# --------------------------------------------------------------------------
# temperature softmax ([SSD-A] names the sampling temperature as what makes
# outcome prediction hard; [SSD-B] part 2 the same for high temperature)
# --------------------------------------------------------------------------
def softmax_t(z, T):
    """Row statistics of softmax(z / T).

    Returns dict(max, lse, argmax, p): max = max z, argmax = lowest index of
    the maximum, lse = ln sum_x exp((z_x - max)/T) and p the distribution.
    Greedy (T not > 0): p = onehot(argmax) and lse = 0.
    """
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z)
    a = int(np.argmax(z))  # first occurrence of the maximum
    if is_greedy(T):
        p = np.zeros_like(z)
        p[a] = 1.0
        return dict(max=m, lse=0.0, argmax=a, p=p)
    e = np.exp((z - m) / T)
    s = np.sum(e)
    return dict(max=m, lse=math.log(s), argmax=a, p=e / s)


# --------------------------------------------------------------------------
# top-F of the draft logits ([SSD-A]: the bonus token is predicted from the
# most likely draft logits)
# --------------------------------------------------------------------------
def topf(z, F):
    """Indices and values of the F largest raw logits, ordered by value
    descending then index ascending (ranking on raw z, not z/T)."""
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    if F <= 0:
        return np.zeros(0, np.int64), np.zeros(0)
    # every top-F element is >= the F-th largest value (library selection),
    # so only those are sorted
    thr = np.partition(z, V - F)[V - F]
    cand = np.nonzero(z >= thr)[0]
    order = cand[np.lexsort((cand, -z[cand]))]
    idx = order[:F]
    return idx.astype(np.int64), z[idx]


# --------------------------------------------------------------------------
# Saguaro sampling sigma_{F,C} ([SSD-B] part 2: the draft's most likely
# tokens are down-weighted by C so the residual mass moves onto them)
# Reading (the formula is lost): w_x = C * q_x on the top-F set S of the raw
# draft logits, w_x = q_x elsewhere, sigma = w / sum(w).
# --------------------------------------------------------------------------
def sigma(z, T, F, C):
    """Returns dict(sigma, S, max, lse, argmax): lse = ln sum_x w'_x with
    w'_x = C^[x in S] exp((z_x - max)/T), the normaliser of sigma relative to
    the row max.  Greedy: sigma = onehot(argmax), lse = 0."""
    z = np.asarray(z, dtype=np.float64)
    st = softmax_t(z, T)
    S, _ = topf(z, F) if F > 0 else (np.zeros(0, np.int64), None)
    if is_greedy(T):
        return dict(sigma=st["p"], S=S, max=st["max"], lse=0.0, argmax=st["argmax"])
    w = np.exp((z - st["max"]) / T)
    w[S] *= C
    tot = np.sum(w)
    return dict(sigma=w / tot, S=S, max=st["max"], lse=math.log(tot), argmax=st["argmax"])


# --------------------------------------------------------------------------
# two-level Gumbel-max sampler (exact: P(block) * P(token | block) = w / sum w)
# --------------------------------------------------------------------------
def _best_two(scores):
    """Index of the best score (lowest index on ties) and the gap to the
    runner-up (inf when there is a single candidate)."""
    i = int(np.argmax(scores))
    if scores.shape[0] < 2:
        return i, math.inf
    rest = np.delete(scores, i)
    return i, float(scores[i] - np.max(rest))


def gsample(w, seed, b, j, tok_stream, blk_stream, blk=BLK):
    """Sample x ~ w / sum(w) with the two-level Gumbel-max rule.

    1. blocks beta = [blk*beta, min(V, blk*beta + blk)), W_beta = sum of w;
    2. beta* = argmax over W_beta > 0 of ln W_beta + G(b, j, beta, blk_stream);
    3. x* = argmax over x in beta*, w_x > 0 of ln w_x + G(b, j, x, tok_stream).
    Ties go to the lower index.  Returns (x*, margin) where margin is the
    smaller of the two stages' best-minus-runner-up score gaps.
    """
    w = np.asarray(w, dtype=np.float64)
    V = w.shape[0]
    nb = (V + blk - 1) // blk
    W = np.array([np.sum(w[k * blk:min(V, k * blk + blk)]) for k in range(nb)])
    cand_b = np.nonzero(W > 0)[0]
    gb = ph.gumbels(seed, b, j, blk_stream, cand_b)
    sb = np.log(W[cand_b]) + gb
    ib, mb = _best_two(sb)
    beta = int(cand_b[ib])
    lo, hi = beta * blk, min(V, beta * blk + blk)
    cand_x = lo + np.nonzero(w[lo:hi] > 0)[0]
    gx = ph.gumbels(seed, b, j, tok_stream, cand_x)
    sx = np.log(w[cand_x]) + gx
    ix, mx = _best_two(sx)
    return int(cand_x[ix]), min(mb, mx)


# --------------------------------------------------------------------------
# draft side: sigma_{F,C} sampling of K tokens plus row statistics and top-F
# --------------------------------------------------------------------------
def draft_sample(zd, T, F, C, seed, F_out=None, blk=BLK, b0=0):
    """zd: [B, K+1, V] fp64 draft logits; T: [B] temperatures.  b0 is the
    batch index of the first sequence (its Philox counters use b0 + b).

    For positions j < K the token x_j ~ sigma_j is drawn with the two-level
    sampler (streams DRAFT_TOKEN / DRAFT_BLOCK); greedy rows take the argmax.
    Row K is not sampled: its statistics and top-F only serve to predict the
    bonus after K acceptances.
    Returns dict(tokens [B,K], q [B,K] = sigma_j(x_j), max/lse/argmax [B,K+1],
    topf_idx/topf_val [B,K+1,F_out], margin [B,K]).
    """
    zd = np.asarray(zd, dtype=np.float64)
    B, K1, V = zd.shape
    K = K1 - 1
    F_out = F if F_out is None else F_out
    out = dict(tokens=np.zeros((B, K), np.int64), q=np.zeros((B, K)),
               max=np.zeros((B, K1)), lse=np.zeros((B, K1)),
               argmax=np.zeros((B, K1), np.int64),
               topf_idx=np.zeros((B, K1, F_out), np.int64),
               topf_val=np.zeros((B, K1, F_out)),
               margin=np.full((B, K), math.inf))
    for b in range(B):
        for j in range(K1):
            sg = sigma(zd[b, j], T[b], F, C)
            out["max"][b, j] = sg["max"]
            out["lse"][b, j] = sg["lse"]
            out["argmax"][b, j] = sg["argmax"]
            ti, tv = topf(zd[b, j], F_out)
            out["topf_idx"][b, j] = ti
            out["topf_val"][b, j] = tv
            if j == K:
                continue
            if is_greedy(T[b]):
                x, mg = sg["argmax"], math.inf
            else:
                x, mg = gsample(sg["sigma"], seed, b0 + b, j, ph.DRAFT_TOKEN, ph.DRAFT_BLOCK, blk)
            out["tokens"][b, j] = x
            out["q"][b, j] = sg["sigma"][x]
            out["margin"][b, j] = mg
    return out


# --------------------------------------------------------------------------
# target side: acceptance test, accepted prefix and bonus token
# ([SSD-A]: accept a prefix of the drafts, then one bonus token that follows
#  all accepted ones; output follows the target distribution;
#  [SSD-B] part 2: on rejection the bonus comes from the residual p - q)
# --------------------------------------------------------------------------
def accept_prob(p, s, x):
    """Exact probability of accepting drafted token x: min(1, p_x / s_x)."""
    if s[x] > 0:
        return min(1.0, p[x] / s[x])
    return 1.0 if p[x] > 0 else 0.0


def residual(p, s):
    """Normalised residual max(0, p - s) / sum; p itself when the sum is 0."""
    r = np.maximum(0.0, p - s)
    t = np.sum(r)
    return r / t if t > 0 else p.copy()


def verify(zt, zd, T, F, C, seed, tokens, blk=BLK, b0=0):
    """zt, zd: [B, K+1, V] fp64; T: [B]; tokens: [B, K] drafted tokens;
    b0: batch index of the first sequence (Philox counters use b0 + b).

    For j = 0..K-1 in order: rho_j = p_j(x_j) / sigma_j(x_j);
    u_j = U(seed, b, j, ACCEPT, idx 0); accept iff u_j < rho_j; stop at the
    first rejection.  k* = number accepted.  Bonus: k* < K -> sample the
    normalised residual max(0, p_k* - sigma_k*) (p_k* if it sums to zero);
    k* = K -> sample p_K.  Both with streams BONUS_TOKEN / BONUS_BLOCK at
    position k*.  Greedy: accept iff x_j = argmax z^t_j; bonus = argmax z^t_k*.
    Tokens outside [0, V) are rejected with p = 0.
    Returns dict(accept_len [B], bonus [B], p [B,K] (all K positions),
    max/lse/argmax [B,K+1] target stats, acc_margin [B,K] (inf where not
    evaluated), bonus_margin [B]).
    """
    zt = np.asarray(zt, dtype=np.float64)
    zd = np.asarray(zd, dtype=np.float64)
    B, K1, V = zt.shape
    K = K1 - 1
    out = dict(accept_len=np.zeros(B, np.int64), bonus=np.zeros(B, np.int64),
               p=np.zeros((B, K)), max=np.zeros((B, K1)), lse=np.zeros((B, K1)),
               argmax=np.zeros((B, K1), np.int64),
               acc_margin=np.full((B, K), math.inf), bonus_margin=np.full(B, math.inf))
    for b in range(B):
        P = [softmax_t(zt[b, j], T[b]) for j in range(K1)]
        for j in range(K1):
            out["max"][b, j] = P[j]["max"]
            out["lse"][b, j] = P[j]["lse"]
            out["argmax"][b, j] = P[j]["argmax"]
        greedy = is_greedy(T[b])
        kstar = K
        decided = False
        for j in range(K):
            x = int(tokens[b, j])
            ok = 0 <= x < V
            pj = P[j]["p"][x] if ok else 0.0
            out["p"][b, j] = pj
            if decided:
                continue
            if not ok:
                acc = False
            elif greedy:
                acc = x == P[j]["argmax"]
            else:
                s = sigma(zd[b, j], T[b], F, C)["sigma"]
                if s[x] > 0:
                    rho = pj / s[x]
                else:
                    rho = math.inf if pj > 0 else 0.0
                u = float(ph.uniforms(seed, b0 + b, j, ph.ACCEPT, np.array([0]))[0])
                acc = u < rho
                out["acc_margin"][b, j] = abs(u - rho)
            if not acc:
                kstar = j
                decided = True
        out["accept_len"][b] = kstar
        if greedy:
            out["bonus"][b] = P[kstar]["argmax"]
            continue
        p = P[kstar]["p"]
        if kstar < K:
            s = sigma(zd[b, kstar], T[b], F, C)["sigma"]
            r = np.maximum(0.0, p - s)
            w = r if np.sum(r) > 0 else p
        else:
            w = p
        x, mg = gsample(w, seed, b0 + b, kstar, ph.BONUS_TOKEN, ph.BONUS_BLOCK, blk)
        out["bonus"][b] = x
        out["bonus_margin"][b] = mg
    return out


# --------------------------------------------------------------------------
# token-tree verification ([SSD-A], closing paragraph of "SSD 如何實現草擬與驗證
# 并行？": SSD combines naturally with token-tree speculation).  The pages give
# no algorithm; the reading is the textbook multi-candidate rule, recursive
# rejection sampling over the drafted children of a node, with the residual
# renormalised after each rejected sibling.  Lossless when the children of a
# node are independent draws from the draft distribution at that node.
# --------------------------------------------------------------------------
def tree_children(parent):
    """Children of every node in index order; parent[0] = -1 (the root) and
    0 <= parent[m] < m for m >= 1."""
    kids = [[] for _ in range(len(parent))]
    for m in range(1, len(parent)):
        kids[parent[m]].append(m)
    return kids


def tree_depth(parent):
    d = [0] * len(parent)
    for m in range(1, len(parent)):
        d[m] = d[parent[m]] + 1
    return d


def verify_tree(zt, zd, T, F, C, seed, parent, tokens, blk=BLK, b0=0):
    """zt, zd: [B, N+1, V] fp64, row n = node n (node 0 is the root, the last
    accepted token's context); parent: [N+1] topology shared by the batch;
    tokens: [B, N+1], tokens[b, m] = token of node m >= 1, drawn from sigma of
    draft row parent[m] (entry 0 unused).

    Walk from the root.  At node n with children m_1 < m_2 < ... (siblings
    i = 0, 1, ...): r = p_n; for each sibling in turn, u = U(seed, b, j = n,
    ACCEPT, idx = i) and accept iff u < r(x) / sigma_n(x) (+inf when sigma_n(x)
    = 0 < r(x), 0 when both are 0 or x is outside [0, V)); on acceptance move
    to that child; on rejection r <- max(0, r - sigma_n), renormalised (kept
    unchanged when it has no mass).  When every sibling is rejected the bonus
    is drawn from r; at a node without children from p_n; both with the
    two-level sampler at (b, j = n, BONUS streams).  Greedy (T not > 0): the
    first sibling whose token is the target row's argmax is accepted, the
    bonus is the argmax of the node where the walk stops.
    Returns dict(accept_len [B] (nodes accepted), last [B] (the node where the
    walk stopped), bonus [B], acc_margin [B, N+1] (|u - ratio| of each
    evaluated node, inf elsewhere), bonus_margin [B])."""
    zt = np.asarray(zt, dtype=np.float64)
    zd = np.asarray(zd, dtype=np.float64)
    B, N1, V = zt.shape
    kids = tree_children(parent)
    out = dict(accept_len=np.zeros(B, np.int64), last=np.zeros(B, np.int64), bonus=np.zeros(B, np.int64),
               acc_margin=np.full((B, N1), math.inf), bonus_margin=np.full(B, math.inf))
    for b in range(B):
        greedy = is_greedy(T[b])
        n, depth = 0, 0
        while True:
            P = softmax_t(zt[b, n], T[b])
            if greedy:
                nxt = next((m for m in kids[n] if int(tokens[b, m]) == P["argmax"]), None)
                if nxt is None:
                    out["bonus"][b] = P["argmax"]
                    break
                n, depth = nxt, depth + 1
                continue
            if not kids[n]:
                x, mg = gsample(P["p"], seed, b0 + b, n, ph.BONUS_TOKEN, ph.BONUS_BLOCK, blk)
                out["bonus"][b], out["bonus_margin"][b] = x, mg
                break
            s = sigma(zd[b, n], T[b], F, C)["sigma"]
            r = P["p"].copy()
            nxt = None
            for i, m in enumerate(kids[n]):
                x = int(tokens[b, m])
                if not 0 <= x < V:
                    rho = 0.0
                elif s[x] > 0:
                    rho = r[x] / s[x]
                else:
                    rho = math.inf if r[x] > 0 else 0.0
                u = float(ph.uniforms(seed, b0 + b, n, ph.ACCEPT, np.array([i]))[0])
                out["acc_margin"][b, m] = abs(u - rho)
                if u < rho:
                    nxt = m
                    break
                nr = np.maximum(0.0, r - s)
                t = np.sum(nr)
                if t > 0:
                    r = nr / t
            if nxt is None:
                x, mg = gsample(r, seed, b0 + b, n, ph.BONUS_TOKEN, ph.BONUS_BLOCK, blk)
                out["bonus"][b], out["bonus_margin"][b] = x, mg
                break
            n, depth = nxt, depth + 1
        out["accept_len"][b] = depth
        out["last"][b] = n
    return out


def acceptance_rate(p, s):
    """alpha = sum_x min(p_x, s_x) ([SSD-B] core-mechanism section names the
    acceptance rate as how well the draft approximates the target; reading of
    its lost formula: the textbook sum of minima, 1 - total variation)."""
    return float(np.sum(np.minimum(p, s)))


# --------------------------------------------------------------------------
# fan-out under a budget ([SSD-B] part 1: the optimal per-depth fan-out F_k
# under budget B is a truncated geometric series, larger at shallow depths
# because the chance of accepting k tokens decays exponentially)
# --------------------------------------------------------------------------
def fanout(Bgt, K, ratio, V):
    """F_k, k = 0..K, proportional to ratio**k with sum exactly Bgt.

    w_k = ratio**k by repeated multiplication from 1.0, S = w_0 + ... + w_K in
    that order, ideal_k = Bgt * w_k / S; F_k = floor(ideal_k) and the
    remaining units go to the largest fractional parts (ties to the smaller
    k).  Each F_k is then capped at V, the excess handed out in ascending k to
    depths still below V.
    """
    w = []
    x = 1.0
    for _ in range(K + 1):
        w.append(x)
        x = x * ratio
    S = 0.0
    for v in w:
        S = S + v
    ideal = [Bgt * v / S for v in w]
    Fk = [int(math.floor(v)) for v in ideal]
    rem = Bgt - sum(Fk)
    order = sorted(range(K + 1), key=lambda k: (-(ideal[k] - math.floor(ideal[k])), k))
    for k in order[:rem]:
        Fk[k] += 1
    excess = 0
    for k in range(K + 1):
        if Fk[k] > V:
            excess += Fk[k] - V
            Fk[k] = V
    for k in range(K + 1):
        if excess == 0:
            break
        give = min(excess, V - Fk[k])
        Fk[k] += give
        excess -= give
    if excess:
        raise ValueError("budget exceeds (K+1)*V")
    return Fk


def depth_probs(alpha, K):
    """a_k = P(k* = k) when each position is accepted independently with
    probability alpha: alpha^k (1 - alpha) for k < K, alpha^K for k = K."""
    return [alpha ** k * (1 - alpha) for k in range(K)] + [alpha ** K]


def optimal_fanout(a, r, Bgt):
    """Maximise sum_k a_k * h(F_k), h(F) = 1 - (1 + F)^-r (chance that the
    bonus lies among F guesses), subject to sum F_k = Bgt, by greedy marginal
    allocation (the objective is separable and concave, so greedy is
    optimal); ties go to the smaller k.  This is the optimisation model under
    which the truncated-geometric shape of [SSD-B] part 1 is checked."""
    F = [0] * len(a)
    for _ in range(Bgt):
        gains = [a[k] * ((1 + F[k]) ** -r - (2 + F[k]) ** -r) for k in range(len(a))]
        k = int(np.argmax(gains))
        F[k] += 1
    return F


def fanout_objective(a, r, F):
    return sum(a[k] * (1 - (1 + F[k]) ** -r) for k in range(len(a)))


def fanout_from_stats(a, h, Bgt):
    """Budget allocation from measured statistics ([SSD-B] part 1: spend the
    cache budget where acceptance stops most often).  a[k]: measured
    P(k* = k); h[k][F]: measured chance that the bonus at depth k is among
    the draft's top-F tokens (F = 0 .. Fmax, h[k][0] = 0).  Each of the Bgt
    slots goes to the depth with the largest gain a[k] (h[k][F_k + 1] -
    h[k][F_k]), ties to the smaller k, depths already at Fmax excluded.
    Maximises sum_k a[k] h[k][F_k] when every h[k] is concave."""
    K1 = len(a)
    Fmax = len(h[0]) - 1
    if Bgt > K1 * Fmax:
        raise ValueError("budget larger than (K+1) Fmax")
    F = [0] * K1
    for _ in range(Bgt):
        best, bk = -math.inf, -1
        for k in range(K1):
            if F[k] < Fmax:
                g = a[k] * (h[k][F[k] + 1] - h[k][F[k]])
                if g > best:
                    best, bk = g, k
        F[bk] += 1
    return F


def fanout_stats_objective(a, h, F):
    return sum(a[k] * h[k][F[k]] for k in range(len(a)))


# --------------------------------------------------------------------------
# speculation cache ([SSD-B] core-mechanism section: the draft fills a
# speculation cache while verification runs, and one lookup follows when the
# outcome returns; [SSD-A]: a hit sends the prepared tokens at once)
# --------------------------------------------------------------------------
def depth_offsets(Fk):
    off = [0]
    for f in Fk:
        off.append(off[-1] + f)
    return off


def build_keys(topf_idx, Fk):
    """keys[b, off_k + i] = i-th best draft token of row k (i < F_k):
    depth-major, then rank."""
    topf_idx = np.asarray(topf_idx)
    B = topf_idx.shape[0]
    off = depth_offsets(Fk)
    keys = np.zeros((B, off[-1]), np.int64)
    for k, f in enumerate(Fk):
        keys[:, off[k]:off[k] + f] = topf_idx[:, k, :f]
    return keys, off


def fallback_tokens(seed, b, K, V):
    """The K random tokens that stand in for sequence b's missed cache entry:
    token i from the FALLBACK stream word at (idx = i, b, j = 0), mapped to
    [0, V) by the high half of word * V.  [SSD-B] part 3: past a critical
    batch size a miss is served by a near-zero-latency speculator such as
    random tokens."""
    if K == 0:
        return np.zeros(0, np.int64)
    w = ph.draw_words(seed, b, 0, ph.FALLBACK, np.arange(K))
    return ph.token_from_word(w, V)


def cache_lookup(keys, off, payload, accept_len, bonus, seed=0, V=0, miss_fill=False):
    """Hit iff bonus is among depth accept_len's keys; slot = the lowest
    such; tokens = payload[slot].  On a miss slot = -1 and the tokens are -1,
    or with miss_fill the sequence's fallback tokens.  An accepted length
    outside [0, K] is a miss."""
    keys = np.asarray(keys)
    payload = np.asarray(payload)
    B = keys.shape[0]
    K = payload.shape[2]
    hit = np.zeros(B, np.int64)
    slot = np.full(B, -1, np.int64)
    toks = np.full((B, K), -1, np.int64)
    for b in range(B):
        k = int(accept_len[b])
        if 0 <= k < len(off) - 1:
            for s in range(off[k], off[k + 1]):
                if keys[b, s] == bonus[b]:
                    hit[b] = 1
                    slot[b] = s
                    toks[b] = payload[b, s]
                    break
        if not hit[b] and miss_fill:
            toks[b] = fallback_tokens(seed, b, K, V)
    return hit, slot, toks


def backoff(p_hit, t_round, t_slow, t_fast, e_acc, e_fast):
    """Which backup speculator serves cache misses ([SSD-B] part 3, reading).

    A round in which any sequence misses waits for the backup, so with the
    chance that the whole batch hits P = prod_b p_b (the pages' observation
    that misses grow with the batch size):
      accurate backup: every sequence yields e_acc tokens, the round takes
                       t_round + (1 - P) t_slow;
      fast backup:     sequence b yields p_b e_acc + (1 - p_b) e_fast tokens,
                       the round takes t_round + (1 - P) t_fast.
    Returns (use_fast, gain) with gain = throughput(fast) / throughput(accurate);
    the fast backup is chosen iff gain > 1 (a tie keeps the accurate one)."""
    p = np.asarray(p_hit, dtype=np.float64)
    B = p.size
    P = float(np.prod(p))
    r_acc = B * e_acc / (t_round + (1.0 - P) * t_slow)
    r_fast = float(np.sum(p * e_acc + (1.0 - p) * e_fast)) / (t_round + (1.0 - P) * t_fast)
    gain = r_fast / r_acc
    return bool(gain > 1.0), gain


def backoff_critical_batch(p, t_round, t_slow, t_fast, e_acc, e_fast):
    """Smallest real batch size B* from which the fast backup wins when every
    sequence hits with chance p (0 < p < 1): equal throughputs at a batch
    miss chance q* = t_round (e_acc - e_mix) / (e_mix t_slow - e_acc t_fast),
    e_mix = p e_acc + (1 - p) e_fast, and 1 - p**B* = q*.  inf when the fast
    backup never wins."""
    e_mix = p * e_acc + (1.0 - p) * e_fast
    den = e_mix * t_slow - e_acc * t_fast
    if den <= 0.0:
        return float("inf")
    q = t_round * (e_acc - e_mix) / den
    if q >= 1.0:
        return float("inf")
    if q <= 0.0:
        return 0.0
    return float(np.log1p(-q) / np.log(p))
