"""Pin checks for the CPU oracle, shared by the pin tests and mutation tests.

Each ``check_*`` function returns the largest deviation it found between the
oracle and something that is not the oracle (a library routine, scalar
brute force, a closed form or an invariant), so that a test can assert it is
small and a mutation test can assert that a planted mistake makes it large.
"""

from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch

import oracle
from oracle import paged_decode as pa
from workloads import make_case, permute_pool, repage


def scatter_into_pages(seqs_k, seqs_v, block_size, num_kv_heads, head_dim, seed,
                       extra_pages=2, fill=0.0):
    """Lay contiguous per-sequence K/V [n_b, Hkv, D] into a shuffled pool.

    This is the inverse direction of the oracle's gather, written
    independently: it walks tokens one by one and writes each into the page
    and slot a fresh random block table assigns.
    """
    rng = np.random.default_rng(seed)
    lens = [k.shape[0] for k in seqs_k]
    npages = [-(-n // block_size) for n in lens]
    P = sum(npages) + extra_pages
    perm = rng.permutation(P)
    W = max(1, max(npages))
    table = np.full((len(lens), W), -1, dtype=np.int64)
    kp = np.full((P, block_size, num_kv_heads, head_dim), fill, dtype=np.float64)
    vp = np.full_like(kp, fill)
    off = 0
    for b, n in enumerate(lens):
        table[b, :npages[b]] = perm[off:off + npages[b]]
        off += npages[b]
        for i in range(n):
            page = table[b, i // block_size]
            kp[page, i % block_size] = seqs_k[b][i]
            vp[page, i % block_size] = seqs_v[b][i]
    return kp, vp, table, np.asarray(lens, dtype=np.int64)


def random_contiguous_case(seed, *, B=3, Tq=2, Hq=8, Hkv=2, D=16, bs=4,
                           lens=(1, 7, 33), scratch=0):
    rng = np.random.default_rng(seed)
    seqs_k = [rng.standard_normal((n, Hkv, D)) for n in lens]
    seqs_v = [rng.standard_normal((n, Hkv, D)) for n in lens]
    q = rng.standard_normal((B, Tq, Hq, D))
    sk = rng.standard_normal((B, scratch, Hkv, D)) if scratch else None
    sv = rng.standard_normal((B, scratch, Hkv, D)) if scratch else None
    kp, vp, table, ctx = scatter_into_pages(seqs_k, seqs_v, bs, Hkv, D, seed + 1)
    return dict(q=q, seqs_k=seqs_k, seqs_v=seqs_v, kp=kp, vp=vp, table=table,
                ctx=ctx, sk=sk, sv=sv, scale=0.3 + 0.05 * (seed % 7))


def check_against_sdpa(c) -> float:
    """Oracle vs torch's float64 scaled_dot_product_attention (GQA) + logsumexp."""
    O, LSE = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"],
                                    c["scale"], scratch_k=c["sk"], scratch_v=c["sv"])
    B, Tq, Hq, D = c["q"].shape
    Hkv = c["kp"].shape[2]
    worst = 0.0
    for b in range(B):
        k = c["seqs_k"][b]
        v = c["seqs_v"][b]
        if c["sk"] is not None:
            k = np.concatenate([k, c["sk"][b]])
            v = np.concatenate([v, c["sv"][b]])
        if k.shape[0] == 0:
            worst = max(worst, float(np.abs(O[b]).max()))
            worst = max(worst, 0.0 if np.all(np.isneginf(LSE[b])) else math.inf)
            continue
        qt = torch.from_numpy(c["q"][b]).permute(1, 0, 2)[None]      # [1, Hq, Tq, D]
        kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()  # [1, Hkv, n, D]
        vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=c["scale"], enable_gqa=True)[0].permute(1, 0, 2).numpy()
        worst = max(worst, float(np.abs(O[b] - ref).max()))
        g = Hq // Hkv
        for t in range(Tq):
            for h in range(Hq):
                s = c["scale"] * np.einsum("d,nd->n", c["q"][b, t, h], k[:, h // g, :])
                worst = max(worst, abs(float(LSE[b, t, h]) - float(
                    scipy.special.logsumexp(s))))
    return worst


def brute_force(q, kp, vp, table, ctx, scale, sk=None, sv=None):
    """Scalar loops with math.fsum over the logical token list."""
    B, Tq, Hq, D = q.shape
    bs, Hkv = kp.shape[1], kp.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, Tq, Hq, D))
    L = np.zeros((B, Tq, Hq))
    for b in range(B):
        for t in range(Tq):
            for h in range(Hq):
                hk = h // g
                keys, vals = [], []
                for i in range(int(ctx[b])):
                    page = int(table[b][i // bs])
                    keys.append([float(x) for x in kp[page][i % bs][hk]])
                    vals.append([float(x) for x in vp[page][i % bs][hk]])
                if sk is not None:
                    for j in range(sk.shape[1]):
                        keys.append([float(x) for x in sk[b][j][hk]])
                        vals.append([float(x) for x in sv[b][j][hk]])
                if not keys:
                    L[b, t, h] = -math.inf
                    continue
                qv = [float(x) for x in q[b][t][h]]
                s = [scale * math.fsum(a * c for a, c in zip(qv, kk)) for kk in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                l = math.fsum(w)
                for d in range(D):
                    O[b, t, h, d] = math.fsum(w[i] * vals[i][d] for i in range(len(w))) / l
                L[b, t, h] = m + math.log(l)
    return O, L


def check_brute_force(c) -> float:
    O, LSE = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"],
                                    c["scale"], scratch_k=c["sk"], scratch_v=c["sv"])
    Ob, Lb = brute_force(c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"],
                         c["sk"], c["sv"])
    finite = np.isfinite(Lb)
    if not np.array_equal(finite, np.isfinite(LSE)):
        return math.inf
    return max(float(np.abs(O - Ob).max()),
               float(np.abs(LSE[finite] - Lb[finite]).max(initial=0.0)))


def check_split_combine(c, splits=(1, 2, 3, 7, 64)) -> float:
    O, LSE = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"],
                                    c["scale"], scratch_k=c["sk"], scratch_v=c["sv"])
    worst = 0.0
    for S in splits:
        Op, Lp = oracle.paged_attention_partials(
            c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"], S,
            scratch_k=c["sk"], scratch_v=c["sv"])
        Oc, Lc = oracle.combine_partials(Op, Lp)
        fin = np.isfinite(LSE)
        if not np.array_equal(fin, np.isfinite(Lc)):
            return math.inf
        worst = max(worst, float(np.abs(Oc - O).max()),
                    float(np.abs(Lc[fin] - LSE[fin]).max(initial=0.0)))
    return worst


def brute_force_partials(q, kp, vp, table, ctx, scale, S, sk=None, sv=None,
                         scratch_mask="none"):
    """Split partials by scalar loops, from the written-out split rule.

    Split s of sequence b owns its logical pages [s*pps, (s+1)*pps) (clipped
    to npages = ceil(ctx_b / bs), pps = ceil(npages / S)), token by token, and
    the last split also owns the scratch tokens (query token t of Tq seeing
    scratch token j of S_tok iff j <= t + S_tok - Tq under the causal mask).
    O_s and LSE_s are the fsum softmax over exactly those tokens; a split with
    none gives (0, -inf).
    """
    B, Tq, Hq, D = q.shape
    bs, Hkv = kp.shape[1], kp.shape[2]
    g = Hq // Hkv
    n_scr = 0 if sk is None else sk.shape[1]
    O = np.zeros((B, Tq, Hq, S, D))
    L = np.full((B, Tq, Hq, S), -math.inf)
    for b in range(B):
        n = int(ctx[b])
        npages = (n + bs - 1) // bs
        pps = (npages + S - 1) // S
        for s in range(S):
            toks = []                       # (page, slot) of every owned paged token
            for pg in range(s * pps, min((s + 1) * pps, npages)):
                for slot in range(bs):
                    if pg * bs + slot < n:
                        toks.append((int(table[b][pg]), slot))
            for t in range(Tq):
                if s == S - 1:
                    vis = n_scr if scratch_mask == "none" else \
                        max(0, min(n_scr, t + n_scr - Tq + 1))
                else:
                    vis = 0
                for h in range(Hq):
                    hk = h // g
                    keys = [[float(x) for x in kp[pg][sl][hk]] for pg, sl in toks]
                    vals = [[float(x) for x in vp[pg][sl][hk]] for pg, sl in toks]
                    keys += [[float(x) for x in sk[b][j][hk]] for j in range(vis)]
                    vals += [[float(x) for x in sv[b][j][hk]] for j in range(vis)]
                    if not keys:
                        continue
                    qv = [float(x) for x in q[b][t][h]]
                    sc = [scale * math.fsum(a * c for a, c in zip(qv, kk)) for kk in keys]
                    m = max(sc)
                    w = [math.exp(x - m) for x in sc]
                    l = math.fsum(w)
                    for d in range(D):
                        O[b, t, h, s, d] = math.fsum(w[i] * vals[i][d] for i in range(len(w))) / l
                    L[b, t, h, s] = m + math.log(l)
    return O, L


def check_partials_brute_force(c, splits=(1, 2, 3, 5, 16), scratch_mask="none") -> float:
    """Every (O_s, LSE_s) of the oracle against the scalar split rule."""
    worst = 0.0
    for S in splits:
        Op, Lp = oracle.paged_attention_partials(
            c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"], S,
            scratch_k=c["sk"], scratch_v=c["sv"], scratch_mask=scratch_mask)
        Ob, Lb = brute_force_partials(c["q"], c["kp"], c["vp"], c["table"], c["ctx"],
                                      c["scale"], S, c["sk"], c["sv"], scratch_mask)
        fin = np.isfinite(Lb)
        if not np.array_equal(fin, np.isfinite(Lp)):
            return math.inf
        worst = max(worst, float(np.abs(Op - Ob).max()),
                    float(np.abs(Lp[fin] - Lb[fin]).max(initial=0.0)))
    return worst


def check_zero_keys_count(seed=5, lens=(0, 1, 5, 16, 17, 40), scratch=3, bs=4) -> float:
    """K = 0: every score is 0, so LSE = ln(number of attended tokens)."""
    rng = np.random.default_rng(seed)
    Hkv, D, Hq = 2, 8, 6
    seqs_k = [np.zeros((n, Hkv, D)) for n in lens]
    seqs_v = [rng.standard_normal((n, Hkv, D)) for n in lens]
    kp, vp, table, ctx = scatter_into_pages(seqs_k, seqs_v, bs, Hkv, D, seed)
    B = len(lens)
    q = rng.standard_normal((B, 2, Hq, D))
    sk = np.zeros((B, scratch, Hkv, D))
    sv = rng.standard_normal((B, scratch, Hkv, D))
    _, LSE = oracle.paged_attention(q, kp, vp, table, ctx, 0.7, scratch_k=sk, scratch_v=sv)
    want = np.log(np.asarray(lens, dtype=np.float64) + scratch)[:, None, None]
    return float(np.abs(LSE - want).max())


def check_needle(seed=9, bs=4, n=23) -> float:
    """One key aligned with every query of its group scores 40; the rest 0.

    O must equal that token's V to within n * e^-40 (< 1e-15 here).
    """
    rng = np.random.default_rng(seed)
    Hkv, g, D = 2, 3, 8
    Hq = Hkv * g
    worst = 0.0
    for star in sorted({0, 1, bs - 1, bs, 2 * bs - 1, n - 2, n - 1}):
        qdir = rng.standard_normal((Hkv, D))
        q = np.repeat(qdir, g, axis=0)[None, None]          # [1, 1, Hq, D]
        scale = 0.5
        k = np.zeros((n, Hkv, D))
        for hk in range(Hkv):
            k[star, hk] = qdir[hk] * (40.0 / (scale * float(qdir[hk] @ qdir[hk])))
        v = rng.standard_normal((n, Hkv, D))
        kp, vp, table, ctx = scatter_into_pages([k], [v], bs, Hkv, D, seed + star)
        O, _ = oracle.paged_attention(q, kp, vp, table, ctx, scale)
        for h in range(Hq):
            worst = max(worst, float(np.abs(O[0, 0, h] - v[star, h // g]).max()))
    return worst


def check_identical_keys(seed=11) -> float:
    """All keys equal: O = mean(V) and LSE = s + ln n."""
    rng = np.random.default_rng(seed)
    Hkv, Hq, D, n, bs = 1, 4, 8, 13, 4
    kk = rng.standard_normal((Hkv, D))
    k = np.repeat(kk[None], n, axis=0)
    v = rng.standard_normal((n, Hkv, D))
    kp, vp, table, ctx = scatter_into_pages([k], [v], bs, Hkv, D, seed)
    q = rng.standard_normal((1, 1, Hq, D))
    scale = 0.4
    O, LSE = oracle.paged_attention(q, kp, vp, table, ctx, scale)
    worst = float(np.abs(O[0, 0] - v[:, 0].mean(axis=0)[None]).max())
    for h in range(Hq):
        s = scale * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0, h], kk[0]))
        worst = max(worst, abs(float(LSE[0, 0, h]) - (s + math.log(n))))
    return worst


def check_single_token(seed=13) -> float:
    """ctx = 1, no scratch: O = v_0 exactly and LSE = s_0."""
    rng = np.random.default_rng(seed)
    Hkv, Hq, D = 2, 4, 8
    k = rng.standard_normal((1, Hkv, D))
    v = rng.standard_normal((1, Hkv, D))
    kp, vp, table, ctx = scatter_into_pages([k], [v], 16, Hkv, D, seed)
    q = rng.standard_normal((1, 3, Hq, D))
    O, LSE = oracle.paged_attention(q, kp, vp, table, ctx, 0.25)
    worst = 0.0
    for t in range(3):
        for h in range(Hq):
            worst = max(worst, float(np.abs(O[0, t, h] - v[0, h // 2]).max()))
            s0 = 0.25 * math.fsum(float(a) * float(b) for a, b in zip(q[0, t, h], k[0, h // 2]))
            worst = max(worst, abs(float(LSE[0, t, h]) - s0))
    return worst


def check_gqa_equals_repeated_mha(seed=17) -> float:
    c = random_contiguous_case(seed, Hq=8, Hkv=2, scratch=2)
    O, LSE = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"],
                                    c["scale"], scratch_k=c["sk"], scratch_v=c["sv"])
    g = 4
    kp = np.repeat(c["kp"], g, axis=2)
    vp = np.repeat(c["vp"], g, axis=2)
    sk = np.repeat(c["sk"], g, axis=2)
    sv = np.repeat(c["sv"], g, axis=2)
    O2, LSE2 = oracle.paged_attention(c["q"], kp, vp, c["table"], c["ctx"], c["scale"],
                                      scratch_k=sk, scratch_v=sv)
    return max(float(np.abs(O - O2).max()), float(np.abs(LSE - LSE2).max()))


def check_query_token_separability(seed=19) -> float:
    c = random_contiguous_case(seed, Tq=3, scratch=1)
    O, LSE = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"],
                                    c["scale"], scratch_k=c["sk"], scratch_v=c["sv"])
    worst = 0.0
    for t in range(3):
        O1, L1 = oracle.paged_attention(c["q"][:, t:t + 1], c["kp"], c["vp"], c["table"],
                                        c["ctx"], c["scale"], scratch_k=c["sk"],
                                        scratch_v=c["sv"])
        worst = max(worst, float(np.abs(O1[:, 0] - O[:, t]).max()),
                    float(np.abs(L1[:, 0] - LSE[:, t]).max()))
    return worst


def check_scratch_as_pages(seed=23) -> float:
    """Scratch tokens behave exactly like extra context tokens at the end."""
    c = random_contiguous_case(seed, scratch=3)
    O, LSE = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"],
                                    c["scale"], scratch_k=c["sk"], scratch_v=c["sv"])
    seqs_k = [np.concatenate([k, c["sk"][b]]) for b, k in enumerate(c["seqs_k"])]
    seqs_v = [np.concatenate([v, c["sv"][b]]) for b, v in enumerate(c["seqs_v"])]
    kp, vp, table, ctx = scatter_into_pages(seqs_k, seqs_v, 4, c["kp"].shape[2],
                                            c["kp"].shape[3], seed + 5)
    O2, LSE2 = oracle.paged_attention(c["q"], kp, vp, table, ctx, c["scale"])
    return max(float(np.abs(O - O2).max()), float(np.abs(LSE - LSE2).max()))


def _run(case):
    return oracle.run_case(case)


def check_pool_permutation_bitexact(seed=29) -> bool:
    case = make_case(batch=3, q_tokens=2, num_q_heads=8, num_kv_heads=2, head_dim=32,
                     block_size=4, ctx=(5, 17, 30), seed=seed, scratch_tokens=2,
                     pool_pages=20, poison=True)
    O, L = _run(case)
    O2, L2 = _run(permute_pool(case, seed + 1))
    return bool(np.array_equal(O, O2) and np.array_equal(L, L2))


def check_page_size_bitexact(seed=31, sizes=(1, 2, 16, 64)) -> bool:
    case = make_case(batch=3, q_tokens=1, num_q_heads=4, num_kv_heads=1, head_dim=16,
                     block_size=4, ctx=(3, 40, 65), seed=seed)
    O, L = _run(case)
    for bs in sizes:
        O2, L2 = _run(repage(case, block_size=bs, seed=seed + bs, pool_extra=1))
        if not (np.array_equal(O, O2) and np.array_equal(L, L2)):
            return False
    return True


# --- causal scratch mask ------------------------------------------------------

def brute_force_causal(q, kp, vp, table, ctx, scale, sk, sv):
    """Scalar loops with math.fsum; scratch token j is a key of query token t
    only when the query's position among the last Tq speculative tokens is at
    or after j's (walked with an explicit position counter, no closed form)."""
    B, Tq, Hq, D = q.shape
    bs, Hkv = kp.shape[1], kp.shape[2]
    S_tok = sk.shape[1]
    g = Hq // Hkv
    O = np.zeros((B, Tq, Hq, D))
    L = np.zeros((B, Tq, Hq))
    for b in range(B):
        for t in range(Tq):
            # Position of query token t among the speculative tokens 0..S_tok-1:
            # the queries are the last Tq of them (positions may be negative
            # when there are fewer scratch tokens than queries).
            pos = S_tok - Tq
            for _ in range(t):
                pos += 1
            for h in range(Hq):
                hk = h // g
                keys, vals = [], []
                for i in range(int(ctx[b])):
                    page = int(table[b][i // bs])
                    keys.append([float(x) for x in kp[page][i % bs][hk]])
                    vals.append([float(x) for x in vp[page][i % bs][hk]])
                for j in range(S_tok):
                    if j > pos:
                        break
                    keys.append([float(x) for x in sk[b][j][hk]])
                    vals.append([float(x) for x in sv[b][j][hk]])
                if not keys:
                    L[b, t, h] = -math.inf
                    continue
                qv = [float(x) for x in q[b][t][h]]
                s = [scale * math.fsum(a * c for a, c in zip(qv, kk)) for kk in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                l = math.fsum(w)
                for d in range(D):
                    O[b, t, h, d] = math.fsum(w[i] * vals[i][d] for i in range(len(w))) / l
                L[b, t, h] = m + math.log(l)
    return O, L


def _max_dev(O, L, Ob, Lb):
    fin = np.isfinite(Lb)
    if not np.array_equal(fin, np.isfinite(L)):
        return math.inf
    if not np.all(np.isneginf(L[~fin])) or np.abs(O[~fin]).max(initial=0.0) != 0.0:
        return math.inf
    return max(float(np.abs(O - Ob).max(initial=0.0)),
               float(np.abs(L[fin] - Lb[fin]).max(initial=0.0)))


def check_causal_brute_force(c) -> float:
    O, L = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"],
                                  scratch_k=c["sk"], scratch_v=c["sv"], scratch_mask="causal")
    Ob, Lb = brute_force_causal(c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"],
                                c["sk"], c["sv"])
    return _max_dev(O, L, Ob, Lb)


def check_causal_against_masked_sdpa(c) -> float:
    """torch's float64 SDPA with an explicit boolean mask built from the
    draft positions (a lower-triangular band placed at the queries' end)."""
    O, L = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"],
                                  scratch_k=c["sk"], scratch_v=c["sv"], scratch_mask="causal")
    B, Tq, Hq, D = c["q"].shape
    S_tok = c["sk"].shape[1]
    worst = 0.0
    for b in range(B):
        n = int(c["ctx"][b])
        k = np.concatenate([c["seqs_k"][b], c["sk"][b]])
        v = np.concatenate([c["seqs_v"][b], c["sv"][b]])
        # Draft grid: rows = the last Tq of S_tok + Tq' positions, columns = the
        # S_tok scratch positions; torch.tril with a diagonal offset places it.
        band = torch.ones(Tq, S_tok, dtype=torch.bool).tril(diagonal=S_tok - Tq)
        mask = torch.cat([torch.ones(Tq, n, dtype=torch.bool), band], dim=1)
        rows_empty = ~mask.any(dim=1)
        qt = torch.from_numpy(c["q"][b]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()
        vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask.clone().masked_fill_(rows_empty[:, None], True),
            scale=c["scale"], enable_gqa=True)[0].permute(1, 0, 2).numpy()
        g = Hq // kt.shape[1]
        for t in range(Tq):
            if bool(rows_empty[t]):
                if not (np.all(O[b, t] == 0.0) and np.all(np.isneginf(L[b, t]))):
                    return math.inf
                continue
            worst = max(worst, float(np.abs(O[b, t] - ref[t]).max()))
            cols = mask[t].numpy()
            for h in range(Hq):
                s = c["scale"] * (k[cols, h // g, :] @ c["q"][b, t, h])
                worst = max(worst, abs(float(L[b, t, h]) - float(scipy.special.logsumexp(s))))
    return worst


def check_causal_invariants(c) -> float:
    """(1) One query token with causal = no mask (it sees every scratch token);
    (2) with S_tok = Tq, query token t under the causal mask equals the
    unmasked decode of that token over the context plus scratch tokens 0..t."""
    kw = dict(scratch_k=c["sk"], scratch_v=c["sv"])
    args = (c["kp"], c["vp"], c["table"], c["ctx"], c["scale"])
    worst = 0.0
    q1 = c["q"][:, -1:]
    Oc, Lc = oracle.paged_attention(q1, *args, scratch_mask="causal", **kw)
    On, Ln = oracle.paged_attention(q1, *args, scratch_mask="none", **kw)
    worst = max(worst, float(np.abs(Oc - On).max()), float(np.abs(Lc - Ln).max()))
    Tq = c["q"].shape[1]
    sk, sv = c["sk"][:, :Tq], c["sv"][:, :Tq]
    Oc, Lc = oracle.paged_attention(c["q"], *args, scratch_k=sk, scratch_v=sv,
                                    scratch_mask="causal")
    for t in range(Tq):
        Ot, Lt = oracle.paged_attention(c["q"][:, t:t + 1], *args, scratch_k=sk[:, :t + 1],
                                        scratch_v=sv[:, :t + 1], scratch_mask="none")
        worst = max(worst, float(np.abs(Oc[:, t:t + 1] - Ot).max()),
                    float(np.abs(Lc[:, t:t + 1] - Lt).max()))
    return worst


def check_causal_split_combine(c, splits=(2, 3, 7)) -> float:
    O, L = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"],
                                  scratch_k=c["sk"], scratch_v=c["sv"], scratch_mask="causal")
    worst = 0.0
    for S in splits:
        Op, Lp = oracle.paged_attention_partials(
            c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"], S,
            scratch_k=c["sk"], scratch_v=c["sv"], scratch_mask="causal")
        Oc, Lc = oracle.combine_partials(Op, Lp)
        worst = max(worst, _max_dev(Oc, Lc, O, L))
    return worst


# --- per-sequence query and scratch counts ---------------------------------------

def check_seq_counts_as_separate_problems(c, q_lens, scratch_lens, mask) -> float:
    """Variable counts equal solving each sequence alone with its arrays cut to
    its counts (padding query rows: O = 0, LSE = -inf)."""
    O, L = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"],
                                  scratch_k=c["sk"], scratch_v=c["sv"], scratch_mask=mask,
                                  q_lens=q_lens, scratch_lens=scratch_lens)
    worst = 0.0
    for b in range(c["q"].shape[0]):
        nq, ns = int(q_lens[b]), int(scratch_lens[b])
        if nq < c["q"].shape[1]:
            if not (np.all(O[b, nq:] == 0.0) and np.all(np.isneginf(L[b, nq:]))):
                return math.inf
        if nq == 0:
            continue
        Ob, Lb = oracle.paged_attention(
            c["q"][b:b + 1, :nq], c["kp"], c["vp"], c["table"][b:b + 1], c["ctx"][b:b + 1],
            c["scale"], scratch_k=c["sk"][b:b + 1, :ns], scratch_v=c["sv"][b:b + 1, :ns],
            scratch_mask=mask)
        worst = max(worst, _max_dev(O[b:b + 1, :nq], L[b:b + 1, :nq], Ob, Lb))
    return worst


def check_seq_counts_brute_force(c, q_lens, scratch_lens, mask) -> float:
    """Scalar brute force with the counts applied by explicit loops."""
    O, L = oracle.paged_attention(c["q"], c["kp"], c["vp"], c["table"], c["ctx"], c["scale"],
                                  scratch_k=c["sk"], scratch_v=c["sv"], scratch_mask=mask,
                                  q_lens=q_lens, scratch_lens=scratch_lens)
    B, Tq, Hq, D = c["q"].shape
    worst = 0.0
    for b in range(B):
        nq, ns = int(q_lens[b]), int(scratch_lens[b])
        sk = c["sk"][b:b + 1, :ns]
        sv = c["sv"][b:b + 1, :ns]
        if nq == 0:
            continue
        if mask == "causal":
            Ob, Lb = brute_force_causal(c["q"][b:b + 1, :nq], c["kp"], c["vp"],
                                        c["table"][b:b + 1], c["ctx"][b:b + 1], c["scale"], sk, sv)
        else:
            Ob, Lb = brute_force(c["q"][b:b + 1, :nq], c["kp"], c["vp"], c["table"][b:b + 1],
                                 c["ctx"][b:b + 1], c["scale"], sk, sv)
        worst = max(worst, _max_dev(O[b:b + 1, :nq], L[b:b + 1, :nq], Ob, Lb))
    return worst
