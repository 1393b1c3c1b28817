"""GPU acceptance statistics on context-free target/draft distributions.

Many independent requests share one fixed pair of logit vectors (so the
acceptance rate alpha = sum_x min(P(x), Q(x)) is the same at every node), draft
tokens are drawn i.i.d. from Q by the test (the drafter), and the HIP walk
decides.  Checks: the CSDN page's E[L] = (1 - alpha^(gamma+1)) / (1 - alpha)
within 1%; the emitted token follows P (chi-square, 16-token vocabulary) for
a chain and for a two-children-per-node tree; alpha = 1 accepts everything;
disjoint supports reject at once.  The first requests are also compared with
the oracle decision by decision.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

pytestmark = pytest.mark.gpu

from parity import log  # noqa: E402
from workloads import trees  # noqa: E402

V = 16


def _pq(seed, sigma_p=1.5, sigma_q=1.0):
    rng = np.random.default_rng(seed)
    pl = (rng.standard_normal(V) * sigma_p).astype(np.float32)
    ql = (pl + rng.standard_normal(V) * sigma_q).astype(np.float32)
    return pl, ql


def _run(parents_one, pl, ql, B, seed, draft_seed, temperature=1.0):
    import tree_attention_verification_02_amd._lib as L
    n = len(parents_one)
    R = B * n
    dev = "cuda"
    rng = np.random.default_rng(draft_seed)
    Q = scipy.special.softmax(ql.astype(np.float64) / temperature)
    toks = rng.choice(V, size=(B, n), p=Q).astype(np.int32)
    toks[:, 0] = 0
    nonleaf = np.zeros(n, dtype=bool)
    nonleaf[parents_one[1:]] = True
    p_rows = np.tile(pl, (R, 1))
    q_rows = np.tile(ql, (R, 1))
    q_rows[np.tile(~nonleaf, B)] = np.nan
    batch = L.Batch(np.arange(0, R + 1, n), np.zeros(B), dev, max_rows=n)
    parents = torch.from_numpy(np.tile(parents_one, B).astype(np.int32)).to(dev)
    tokens = torch.from_numpy(toks.reshape(-1)).to(dev)
    p_t = torch.from_numpy(p_rows).to(dev)
    q_t = torch.from_numpy(q_rows).to(dev)
    out = L.AcceptOut(torch.empty(B, dtype=torch.int32, device=dev),
                      torch.empty((B, n), dtype=torch.int32, device=dev),
                      torch.empty((B, n), dtype=torch.int32, device=dev),
                      flags=torch.empty(B, dtype=torch.int32, device=dev))
    ws = torch.empty(L.spec_accept_workspace_bytes(batch, V), dtype=torch.uint8, device=dev)
    L.spec_accept_sample(batch, parents, tokens, p_t, q_t if temperature > 0 else None, V,
                         temperature, seed, 0, out, ws)
    torch.cuda.synchronize()
    return (out.accept_len.cpu().numpy(), out.tokens.cpu().numpy(), out.path.cpu().numpy(),
            out.flags.cpu().numpy(), toks)


def _oracle_match(parents_one, pl, ql, toks, alen, path, tokens_out, flags, seed, count):
    from oracle import accept as OA
    n = len(parents_one)
    plr = np.tile(pl.astype(np.float64), (n, 1))
    qlr = np.tile(ql.astype(np.float64), (n, 1))
    for b in range(count):
        r = OA.accept_request(parents_one, toks[b], plr, qlr, 1.0, seed, 0, b)
        r["result"].check_outputs(alen[b], path[b], tokens_out[b], flags=flags[b],
                                  what=f"request {b}")


def _chi2_p(samples, P):
    counts = np.bincount(samples, minlength=V).astype(np.float64)
    exp = P * len(samples)
    keep = exp >= 5
    c = np.append(counts[keep], counts[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        c, e = c[:-1], e[:-1]
    return scipy.stats.chisquare(c, e).pvalue


def test_expected_length_chain_gamma8():
    pl, ql = _pq(0)
    P = scipy.special.softmax(pl.astype(np.float64))
    Q = scipy.special.softmax(ql.astype(np.float64))
    alpha = np.minimum(P, Q).sum()
    gamma = 8
    B = 100000
    alen, toks_out, path, flags, toks = _run(trees.chain(gamma), pl, ql, B, seed=3, draft_seed=4)
    Lm = (alen + 1).mean()
    expect = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    log(f"[stats] E[L] gpu {Lm:.4f} closed form {expect:.4f} alpha {alpha:.4f}")
    assert abs(Lm - expect) / expect < 0.01
    assert (flags == 0).all()
    _oracle_match(trees.chain(gamma), pl, ql, toks, alen, path, toks_out, flags, 3, 300)


def test_lossless_chain_and_tree_chi_square():
    for parents_one, seed in ((trees.chain(4), 11), (trees.cartesian((2, 2)), 12)):
        pl, ql = _pq(6, sigma_q=1.5)
        P = scipy.special.softmax(pl.astype(np.float64))
        alen, toks_out, path, flags, toks = _run(parents_one, pl, ql, 100000, seed=seed,
                                                 draft_seed=seed + 1)
        pv = _chi2_p(toks_out[:, 0], P)
        log(f"[stats] chi-square p-value {pv:.4f} for tree of {len(parents_one)} rows")
        assert pv > 1e-3
        _oracle_match(parents_one, pl, ql, toks, alen, path, toks_out, flags, seed, 300)


def test_alpha_one_and_disjoint_support():
    pl, _ = _pq(4)
    alen, _, path, _, _ = _run(trees.chain(6), pl, pl.copy(), 2000, seed=1, draft_seed=2)
    assert (alen == 6).all()
    pl = np.full(V, -30.0, dtype=np.float32)
    pl[:8] = np.log(np.arange(1, 9)).astype(np.float32)
    ql = np.full(V, -30.0, dtype=np.float32)
    ql[8:] = 0.0
    alen, toks_out, _, _, _ = _run(trees.chain(5), pl, ql, 20000, seed=5, draft_seed=6)
    assert (alen == 0).all()
    P = scipy.special.softmax(pl.astype(np.float64))
    assert _chi2_p(toks_out[:, 0], P) > 1e-3


def test_greedy_batch_matches_oracle():
    from oracle import accept as OA
    rng = np.random.default_rng(8)
    parents_one = trees.k_schedule((3, 2, 1))
    n = len(parents_one)
    import tree_attention_verification_02_amd._lib as L
    B = 500
    pl = rng.standard_normal((B * n, V)).astype(np.float32)
    # make ties in some rows: lowest index must win
    pl[::7, 3] = pl[::7].max(axis=1) + 1.0
    pl[::7, 9] = pl[::7, 3]
    toks = np.argmax(pl.reshape(B, n, V), axis=2)
    par = np.tile(parents_one, B)
    # tokens of row c: its parent's argmax half of the time, else random
    t = np.zeros(B * n, dtype=np.int32)
    for r in range(B * n):
        if par[r] >= 0:
            u = (r // n) * n + par[r]
            t[r] = toks.reshape(-1)[u] if rng.random() < 0.6 else rng.integers(V)
    dev = "cuda"
    batch = L.Batch(np.arange(0, B * n + 1, n), np.zeros(B), dev, max_rows=n)
    out = L.AcceptOut(torch.empty(B, dtype=torch.int32, device=dev),
                      torch.empty((B, n), dtype=torch.int32, device=dev),
                      torch.empty((B, n), dtype=torch.int32, device=dev))
    ws = torch.empty(L.spec_accept_workspace_bytes(batch, V), dtype=torch.uint8, device=dev)
    L.spec_accept_sample(batch, torch.from_numpy(par.astype(np.int32)).to(dev),
                         torch.from_numpy(t).to(dev), torch.from_numpy(pl).to(dev), None, V, 0.0,
                         0, 0, out, ws)
    torch.cuda.synchronize()
    alen = out.accept_len.cpu().numpy()
    tk = out.tokens.cpu().numpy()
    for b in range(B):
        r = OA.accept_request(parents_one, t[b * n:(b + 1) * n], pl[b * n:(b + 1) * n].astype(np.float64),
                              None, 0.0, 0, 0, b)
        assert alen[b] == r["accept_len"]
        assert list(tk[b, :len(r["tokens"])]) == r["tokens"]
