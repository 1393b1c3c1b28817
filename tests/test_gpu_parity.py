"""GPU parity: the HIP library against the oracle on seeded workloads.

Reduced sizes span several 64-key tiles, several key splits and ragged tails;
full sizes are the five stated workloads, checked on every request (every
row and head for attention).  Tolerances: masks, commits,
paths and tokens bit-exact (near-threshold sampling decisions are reported,
not failed); attention max |d| <= 1e-2 for bf16 inputs (1e-4 for fp32);
child probabilities within 1e-5 relative.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import attention as OAt  # noqa: E402
from parity import (ATTN_TOL, bits_equal, check_accept, check_attention, check_commit,  # noqa: E402
                    check_mask, log, make, request_slice, run_step)

SMALL = {
    "toy": dict(),
    "chain8-small": dict(L=300, V=5000),
    "chain8-d64": dict(L=333, V=4000, D=64, Hq=8, Hkv=8),
    "medusa-small": dict(L=200, V=3000, Hq=4, Hkv=4),
    "medusa-256rows": dict(L=150, V=2000, Hq=2, Hkv=2, tree=("cartesian", (5, 5, 9))),
    "specinfer-small": dict(B=3, L=700, Hq=16, Hkv=2, V=6000),
    "dynamic-small": dict(B=6, L=("uniform", 30, 700), V=5000),
    "dynamic-contig": dict(B=5, L=("uniform", 0, 300), V=4004, kv_layout="contig"),
    "specinfer-empty-prefix": dict(B=2, L=0, Hq=8, Hkv=2, V=2048),
    # more than 256 query rows per (request, KV head): the 4-wave wide kernel
    "specinfer-wide-paged-d64": dict(B=2, L=900, Hq=16, Hkv=2, D=64, V=3000, kv_layout="paged"),
    "dynamic-wide-mixed": dict(B=7, L=("uniform", 0, 900), Hq=32, Hkv=2, V=3000),
    "medusa-wide-3blocks": dict(L=260, V=2000, Hq=16, Hkv=1, D=64, tree=("cartesian", (2, 3, 4))),
}
BASE = {"toy": "toy", "chain8-small": "chain8", "chain8-d64": "chain8", "medusa-small": "medusa",
        "medusa-256rows": "medusa", "specinfer-small": "specinfer", "dynamic-small": "dynamic",
        "dynamic-contig": "dynamic", "specinfer-empty-prefix": "specinfer",
        "specinfer-wide-paged-d64": "specinfer", "dynamic-wide-mixed": "dynamic",
        "medusa-wide-3blocks": "medusa"}


@pytest.fixture(scope="module")
def lib():
    import tree_attention_verification_02_amd as T
    assert torch.cuda.is_available()
    return T


@pytest.mark.parametrize("case", list(SMALL))
def test_small_sampling(lib, case):
    w = make(BASE[case], **SMALL[case])
    snap = w.k_cache.clone()
    vs = run_step(w, temperature=1.0, seed=0, step=0)
    check_mask(w, vs)
    worst = check_attention(w, vs)
    log(f"[parity] {case}: attention max|d| = {worst:.3e}")
    check_accept(w, vs, 1.0, 0, 0)
    check_commit(w, vs)
    # the library never writes below a request's prefix length
    if w.kv_layout == "contig":
        for b in range(w.B):
            L = int(w.prefix_len[b])
            assert bits_equal(w.k_cache[b, :, :L], snap[b, :, :L])


# Batches of 8 requests and more run with the walks first in the grid: each
# walk takes a node's statistics when it reaches the node, while the
# statistics of deeper rows still stream.  Chains make a walk wait at every
# level; wide trees make it pass over residuals between the waits.
WALKS_FIRST = {
    "chain8-batch12": ("chain8", dict(B=12, L=100, V=3000, Hq=4, Hkv=4)),
    "medusa-batch8": ("medusa", dict(B=8, L=64, V=2000, Hq=4, Hkv=4, tree=("cartesian", (2, 3, 2)))),
    "dynamic-batch20": ("dynamic", dict(B=20, L=("uniform", 8, 200), V=5000, Hq=4, Hkv=1)),
}


@pytest.mark.parametrize("case", list(WALKS_FIRST))
@pytest.mark.parametrize("T,seed,step", [(1.0, 0, 0), (0.3, 4, 1), (2.0, 9, 3)])
def test_walks_first_batches(lib, case, T, seed, step):
    base, kw = WALKS_FIRST[case]
    w = make(base, **kw)
    vs = run_step(w, temperature=T, seed=seed, step=step, commit=False)
    check_accept(w, vs, T, seed, step)


@pytest.mark.parametrize("case", ["chain8-small", "medusa-small", "dynamic-small", "toy"])
def test_small_greedy(lib, case):
    w = make(BASE[case], **SMALL[case])
    vs = run_step(w, temperature=0.0)
    check_accept(w, vs, 0.0, 0, 0)
    check_commit(w, vs)


def _accept_with_knobs(vs, T, seed, step, max_slices=0, max_spins=-1):
    import tree_attention_verification_02_amd._lib as L
    w = vs.w
    L.spec_accept_sample_walk_knobs(vs.batch, vs.parents, vs.tokens, w.p_logits, w.q_logits,
                                    w.V, T, seed, step, vs.acc, vs.acc_ws,
                                    max_slices=max_slices, max_spins=max_spins)
    torch.cuda.synchronize()


@pytest.mark.parametrize("slices", [1, 3, 64])
def test_walk_slices(lib, slices):
    """The walk gives the same result however many workgroups share a request."""
    w = make("dynamic", B=5, L=("uniform", 30, 300), V=20000)
    vs = run_step(w, temperature=1.0, seed=2, step=1, commit=False)
    _accept_with_knobs(vs, 1.0, 2, 1, max_slices=slices)
    check_accept(w, vs, 1.0, 2, 1)


def test_walk_barrier_timeout_is_reported(lib):
    """A walk meeting that does not complete in time (forced from the host:
    max_spins = 0, so a workgroup gives up at its first poll unless every
    workgroup of its request has already arrived) reports the request as
    accept_len = -1, path and tokens -1, SPEC_FLAG_SYNC_TIMEOUT; every other
    request is exact; every kernel ends; the next ordinary call is exact."""
    import tree_attention_verification_02_amd._lib as L
    w = make("dynamic", B=16, L=("uniform", 30, 300), V=50000)
    vs = run_step(w, temperature=1.0, seed=5, step=2, commit=False)
    ref = check_accept(w, vs, 1.0, 5, 2)
    _accept_with_knobs(vs, 1.0, 5, 2, max_slices=8, max_spins=0)
    alen = vs.acc.accept_len.cpu().numpy()
    flags = vs.acc.flags.cpu().numpy()
    path = vs.acc.path.cpu().numpy()
    toks = vs.acc.tokens.cpu().numpy()
    amask = vs.acc.accept_mask.cpu().numpy()
    timed_out = 0
    for b in range(w.B):
        o, e = request_slice(w, b)
        if flags[b] & L.SPEC_FLAG_SYNC_TIMEOUT:
            timed_out += 1
            assert alen[b] == -1 and (path[b] == -1).all() and (toks[b] == -1).all()
            assert (amask[o:e] == 0).all()
        else:
            ref[b]["result"].check_outputs(alen[b], path[b], toks[b], flags=flags[b],
                                           accept_mask=amask[o:e], what=f"request {b}")
    log(f"[parity] forced walk timeouts: {timed_out} of {w.B} requests")
    assert timed_out > 0
    vs.accept()
    torch.cuda.synchronize()
    check_accept(w, vs, 1.0, 5, 2)


def test_zero_residual_branch(lib):
    """The residual norm(max(0, p - q)) of the CSDN page's section 7.1 has no
    mass when the target and draft distributions agree.  At the root of every
    other request the draft row is set to the target row and the first
    child's token gets logit -1e4 in both (probability exactly 0): that child
    is rejected for every coin, the residual mass is exactly 0, and R is kept
    (SPEC_FLAG_ZERO_RESIDUAL).  The next sibling's test r * Q(x) < P(x) = Q(x)
    then passes for every coin.  Everything is compared with the oracle."""
    import tree_attention_verification_02_amd._lib as L
    w = make("dynamic", B=8, L=("uniform", 30, 300), V=6000)
    planted = []
    for b in range(0, w.B, 2):
        o, e = request_slice(w, b)
        kids = [c for c in range(1, e - o) if int(w.parents[o + c]) == 0]
        if not kids:
            continue
        w.q_logits[o].copy_(w.p_logits[o])
        x = int(w.tokens[o + kids[0]])
        w.p_logits[o, x] = -1e4
        w.q_logits[o, x] = -1e4
        planted.append((b, kids))
    assert len(planted) >= 3
    vs = run_step(w, temperature=1.0, seed=6, step=0, commit=False)
    ref = check_accept(w, vs, 1.0, 6, 0, max_flagged=0)
    flags = vs.acc.flags.cpu().numpy()
    path = vs.acc.path.cpu().numpy()
    for b, kids in planted:
        res = ref[b]["result"]
        assert res.zero_residual and res.first_flag() in (None, len(res.decisions) - 1), b
        assert flags[b] & L.SPEC_FLAG_ZERO_RESIDUAL, (b, flags[b])
        o = int(w.row_offsets[b])
        x0 = int(w.tokens[o + kids[0]])
        later = [c for c in kids[1:] if int(w.tokens[o + c]) != x0]
        if later:                       # first sibling with another token: always accepted
            assert path[b, 1] == later[0], (b, path[b])
    log(f"[parity] zero residual: {len(planted)} requests planted, all flagged and exact")


@pytest.mark.parametrize("case,T,seed,step", [("dynamic-small", 0.7, 5, 3),
                                              ("medusa-small", 1.6, 1, 9),
                                              ("specinfer-small", 0.05, 3, 1),
                                              ("chain8-small", 4.0, 2, 2)])
def test_small_other_temperatures(lib, case, T, seed, step):
    w = make(BASE[case], **SMALL[case])
    vs = run_step(w, temperature=T, seed=seed, step=step)
    check_accept(w, vs, T, seed, step)


@pytest.mark.parametrize("mode", ["sample", "topk", "greedy"])
def test_ragged_vocab_with_padded_rows(lib, mode):
    """vocab = 4001 inside rows of 4004 floats whose padding holds NaN: the
    last float4 of every row is partly outside the vocabulary and must be
    masked, never read as a logit.  Checked against the oracle on the
    unpadded rows."""
    import tree_attention_verification_02_amd._lib as L
    from oracle import accept as OA
    V, LD = 4001, 4004
    w = make("dynamic", B=5, L=64, V=V, Hq=4, Hkv=1,
             **({"draft": "topk"} if mode == "topk" else {}))
    dev = "cuda"
    R = w.R
    pl = torch.full((R, LD), float("nan"), dtype=torch.float32, device=dev)
    ql = torch.full((R, LD), float("nan"), dtype=torch.float32, device=dev)
    pl[:, :V] = w.p_logits
    ql[:, :V] = torch.nan_to_num(w.q_logits, nan=0.0)
    batch = L.Batch(w.row_offsets, w.prefix_len, dev)
    S = batch.c.max_rows
    out = L.AcceptOut(torch.empty(w.B, dtype=torch.int32, device=dev),
                      torch.empty((w.B, S), dtype=torch.int32, device=dev),
                      torch.empty((w.B, S), dtype=torch.int32, device=dev),
                      child_p=torch.empty(R, dtype=torch.float32, device=dev),
                      flags=torch.empty(w.B, dtype=torch.int32, device=dev))
    ws = torch.empty(L.spec_accept_workspace_bytes(batch, V), dtype=torch.uint8, device=dev)
    par = torch.from_numpy(w.parents.astype(np.int32)).to(dev)
    tok = torch.from_numpy(w.tokens.astype(np.int32)).to(dev)
    T = 0.0 if mode == "greedy" else 1.0
    if mode == "topk":
        L.spec_accept_topk(batch, par, tok, pl, V, T, 4, 0, out, ws, logits_ld=LD)
    else:
        L.spec_accept_sample(batch, par, tok, pl, ql if T > 0 else None, V, T, 4, 0, out, ws,
                             logits_ld=LD)
    torch.cuda.synchronize()
    alen = out.accept_len.cpu().numpy()
    toks = out.tokens.cpu().numpy()
    path = out.path.cpu().numpy()
    cp = out.child_p.cpu().numpy()
    assert np.isfinite(cp[np.asarray(w.parents) >= 0]).all()
    for b in range(w.B):
        o, e = request_slice(w, b)
        p64 = w.p_logits[o:e].double().cpu().numpy()
        q64 = torch.nan_to_num(w.q_logits[o:e], nan=0.0).double().cpu().numpy()
        if mode == "topk":
            r = OA.accept_request_topk(w.parents[o:e], w.tokens[o:e], p64, T, 4, 0, b)
        else:
            r = OA.accept_request(w.parents[o:e], w.tokens[o:e], p64, q64 if T > 0 else None, T,
                                  4, 0, b)
        r["result"].check_outputs(alen[b], path[b], toks[b], what=f"request {b}")


def test_fp32_output_of_bf16_path(lib):
    w = make("specinfer", **SMALL["specinfer-small"])
    vs = run_step(w, out_dtype=torch.float32)
    worst = check_attention(w, vs, tol=5e-3)
    log(f"[parity] fp32-out bf16 path max|d| = {worst:.3e}")


def test_large_batch_in_request_order(lib):
    """More than 512 requests: the attention grid keeps request order (no
    longest-first phase), and one workspace holds every request's rows."""
    w = make("dynamic", B=600, L=("uniform", 20, 400), V=1500)
    vs = run_step(w, temperature=1.0, seed=3, step=2)
    check_mask(w, vs)
    req = [0, 1, 255, 511, 512, 598, 599]
    worst = check_attention(w, vs, requests=req)
    log(f"[parity] B=600: attention max|d| = {worst:.3e} on requests {req}")
    check_accept(w, vs, 1.0, 3, 2)
    check_commit(w, vs, requests=req, heads=[0, w.Hkv - 1])


def test_deterministic(lib):
    w = make("dynamic", **SMALL["dynamic-small"])
    a = run_step(w, commit=False)
    out1 = a.attn_out.clone()
    acc1 = [t.clone() for t in (a.acc.accept_len, a.acc.path, a.acc.tokens, a.acc.child_p)]
    a.run(commit=False)
    torch.cuda.synchronize()
    assert bits_equal(out1, a.attn_out)
    for x, y in zip(acc1, (a.acc.accept_len, a.acc.path, a.acc.tokens, a.acc.child_p)):
        assert bits_equal(x, y)


@pytest.mark.parametrize("fill", [0, 3, -1])
def test_attention_workspace_contents_do_not_matter(lib, fill):
    """Mixed-length batches hand out their work items through a counter in
    the workspace; whatever the workspace holds before a call (zeros, a small
    in-range value, all ones), the output is the same bits and matches the
    oracle."""
    w = make("dynamic", **SMALL["dynamic-wide-mixed"])
    a = run_step(w, commit=False)
    ref = a.attn_out.clone()
    a.attn_ws.view(torch.int32)[: a.attn_ws.numel() // 4].fill_(fill)
    a.attention()
    torch.cuda.synchronize()
    assert bits_equal(ref, a.attn_out)
    check_attention(w, a)
    a.attention()                       # the counter is reset for the next call
    torch.cuda.synchronize()
    assert bits_equal(ref, a.attn_out)


def test_mixed_batch_heavy_units_and_long_prefix(lib):
    """A mixed-length batch that exercises the planner's corners: a 256-row
    tree with G=4 (1024 query rows: four row blocks of heavy units, which get
    shorter splits), a 40000-key prefix (many splits, tail merged into the
    previous split when short), an empty prefix and a single-row request."""
    from workloads import trees as TR
    big = TR.cartesian((5, 5, 9))                       # 256 rows
    mid = TR.k_schedule((3, 2, 2, 1, 1))                # 46 rows
    w = make("dynamic", B=4, L=[40000, 0, 5000, 777], Hq=8, Hkv=2, V=3000,
             tree=("given", [big, mid, np.array([-1]), TR.chain(8)]))
    # fp32 output: the empty-prefix request averages a handful of values of
    # magnitude up to ~4, where bf16 output rounding alone approaches 1e-2
    vs = run_step(w, temperature=1.0, seed=2, step=5, out_dtype=torch.float32)
    check_mask(w, vs)
    worst = check_attention(w, vs, requests=[0, 1, 2, 3])
    log(f"[parity] mixed heavy batch: attention max|d| = {worst:.3e}")
    check_accept(w, vs, 1.0, 2, 5)
    check_commit(w, vs, heads=[0, 1])


def test_device_side_tree_validation(lib):
    import tree_attention_verification_02_amd._lib as L
    w = make("dynamic", **SMALL["dynamic-small"])
    from tree_attention_verification_02_amd.pipeline import VerifyStep
    vs = VerifyStep(w)
    bad = vs.parents.clone()
    o = int(w.row_offsets[2])
    bad[o + 3] = 7                     # parent not before the row
    bad[int(w.row_offsets[4])] = 0     # root without -1
    vs.parents = bad
    vs.build_mask()
    vs.accept()
    torch.cuda.synchronize()
    err = vs.err_row.cpu().numpy()
    assert err[2] == 3 and err[4] == 0
    assert (err[[0, 1, 3, 5]] == -1).all()
    m = vs.mask.cpu().numpy()
    assert (m[o:int(w.row_offsets[3])] == 0).all()
    flags = vs.acc.flags.cpu().numpy()
    alen = vs.acc.accept_len.cpu().numpy()
    assert flags[2] == L.SPEC_FLAG_BAD_TREE and alen[2] == -1
    assert flags[4] == L.SPEC_FLAG_BAD_TREE and alen[4] == -1
    # the child probabilities of an invalid tree are NaN (T > 0)
    assert vs.temperature > 0
    cp = vs.acc.child_p.cpu().numpy()
    cq = vs.acc.child_q.cpu().numpy()
    for b in (2, 4):
        lo, hi = int(w.row_offsets[b]), int(w.row_offsets[b + 1])
        assert np.isnan(cp[lo:hi]).all() and np.isnan(cq[lo:hi]).all()


def test_path_truncation_flag(lib):
    import tree_attention_verification_02_amd._lib as L
    w = make("chain8", L=64, V=512, Hq=2, Hkv=2, q_sigma=0.0)   # q = p: every draft accepted
    vs = run_step(w, path_stride=4, commit=False)
    assert int(vs.acc.flags[0]) == L.SPEC_FLAG_PATH_TRUNCATED
    assert int(vs.acc.accept_len[0]) == 3
    assert vs.acc.path[0].tolist() == [0, 1, 2, 3]
    assert vs.acc.tokens[0].tolist()[3] == -1


def test_commit_adversarial_paths(lib):
    """In-place compaction with overlapping source/destination slots."""
    w = make("medusa", **SMALL["medusa-small"])
    from tree_attention_verification_02_amd.pipeline import VerifyStep
    import tree_attention_verification_02_amd._lib as L
    vs = VerifyStep(w, path_stride=8)
    vs.append()
    # hand-made accepted paths: root->1->(child of 1)->... in the Cartesian tree
    from oracle import tree as OT
    kids = OT.children(w.parents)
    p = [0, 2, kids[2][4], kids[kids[2][4]][6]]
    vs.acc.accept_len[0] = len(p) - 1
    vs.acc.path[0, :] = -1
    vs.acc.path[0, :len(p)] = torch.tensor(p, dtype=torch.int32)
    vs.commit()
    torch.cuda.synchronize()
    check_commit(w, vs)
    # a chain-prefix path is the identity
    w2 = make("chain8", L=100, V=512, Hq=2, Hkv=2)
    vs2 = VerifyStep(w2, path_stride=9)
    vs2.append()
    before = w2.k_cache.clone()
    vs2.acc.accept_len[0] = 4
    vs2.acc.path[0, :] = torch.tensor([0, 1, 2, 3, 4, -1, -1, -1, -1], dtype=torch.int32)
    vs2.commit()
    torch.cuda.synchronize()
    assert bits_equal(before, w2.k_cache)
    # an inconsistent path is refused with new_len = -1 and no write
    vs2.acc.path[0, :5] = torch.tensor([0, 2, 1, 3, 4], dtype=torch.int32)
    vs2.commit()
    torch.cuda.synchronize()
    assert int(vs2.new_len[0]) == -1
    assert bits_equal(before, w2.k_cache)
    del L


FULL = ["toy", "chain8", "medusa", "specinfer", "dynamic", "lookahead"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(lib, name):
    """Every request of every stated workload at full size: masks, attention
    of every row and head, acceptance and the committed cache."""
    w = make(name)
    vs = run_step(w, temperature=1.0, seed=0, step=0)
    check_mask(w, vs)
    worst = check_attention(w, vs)
    log(f"[parity] full {name}: attention max|d| = {worst:.3e} on all {w.B} requests")
    check_accept(w, vs, 1.0, 0, 0)
    check_commit(w, vs, heads=[0, w.Hkv - 1])
    alen = vs.acc.accept_len.cpu().numpy()
    log(f"[parity] full {name}: mean accepted drafts {alen.mean():.3f}")


@pytest.mark.parametrize("name", ["toy", "chain8", "medusa", "specinfer", "dynamic"])
def test_full_size_greedy_and_seed1(lib, name):
    w = make(name)
    vs = run_step(w, temperature=0.0, commit=False)
    check_accept(w, vs, 0.0, 0, 0)
    vs = run_step(w, temperature=1.0, seed=1, step=0, commit=False)
    check_accept(w, vs, 1.0, 1, 0)


@pytest.mark.parametrize("kind", ["lookahead", "random"])
def test_caller_supplied_masks(lib, kind):
    """Any visibility of the new rows, packed by the caller: the survey page's
    lookahead decoding mask (two causal branches sharing the current token,
    W=5, N=4, G=5: 30 rows) and arbitrary bits (rows may see later rows)."""
    from oracle import tree as OTr
    from workloads import masks
    from tree_attention_verification_02_amd.pipeline import VerifyStep
    if kind == "lookahead":
        w = make("chain8", B=3, tree=("chain", 29), L=("uniform", 0, 400), V=2000, Hq=16, Hkv=2)
    else:
        w = make("dynamic", **SMALL["dynamic-small"])
    vs = VerifyStep(w)
    vs.build_mask()
    rng = np.random.default_rng(7)
    words = vs.batch.words
    new = np.zeros((w.R, words), dtype=np.uint64)
    vis = {}
    for b in range(w.B):
        o, e = request_slice(w, b)
        n = e - o
        vis[b] = (masks.lookahead_visibility(5, 4, 5) if kind == "lookahead"
                  else masks.random_visibility(rng, n, 0.3))
        assert vis[b].shape == (n, n)
        new[o:e] = OTr.pack_words(vis[b], words)
    vs.mask.copy_(torch.from_numpy(new.view(np.int64)).to(vs.mask.device))
    vs.append()
    vs.attention()
    torch.cuda.synchronize()
    out = vs.attn_out.detach().to("cpu", torch.float64).numpy()
    worst = 0.0
    for b in range(w.B):
        o, e = request_slice(w, b)
        kp, vp = w.prefix_kv(b)
        q = w.q[o:e].detach().to("cpu", torch.float64).numpy()
        kt = w.k_new[o:e].detach().to("cpu", torch.float64).numpy()
        vt = w.v_new[o:e].detach().to("cpu", torch.float64).numpy()
        ref = OAt.masked_attention(q, kp, vp, kt, vt, vis[b], scale=1.0 / np.sqrt(w.D))
        err = float(np.abs(out[o:e] - ref).max())
        worst = max(worst, err)
        assert err <= ATTN_TOL, f"{kind} request {b}: max |d| = {err}"
    log(f"[parity] {kind} masks: attention max|d| = {worst:.3e}")
