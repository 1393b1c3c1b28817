"""Seeded synthetic inputs for the verify step.

One ``Workload`` holds everything a verify step consumes: the flattened draft
trees (parents in local row numbering, row offsets), the KV prefix lengths,
the draft tokens, queries, the tree's own K/V rows, the KV cache (contiguous
``[B][Hkv][capacity][D]`` or paged ``[blocks][Hkv][16][D]`` with a block
table), and the target / draft logits.

This module contains no part of the verify method: no mask, attention,
softmax, acceptance or commit arithmetic.  It only draws random numbers with
the shapes and distributions of the five workloads and lays them out.  Large
tensors are drawn with a seeded ``torch.Generator`` on the requested device
(the GPU when one is used, so a 2 GB paged cache is made in milliseconds);
``host()`` hands float64 / int copies to anyone who needs them on the CPU.

Draft tokens are sampled the way a drafter would: child ``c`` of row ``u`` is
a draw from softmax(q_logits[u] / T) with T = 1, taken with the Gumbel-max
trick (argmax of logits plus Gumbel noise), independently per child.  With
``draft="topk"`` the children are the drafter's top choices instead: the
i-th child of ``u`` (in row order) gets the i-th largest entry of
q_logits[u] (a stable sort, so equal logits keep vocabulary order).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np
import torch

from . import masks, trees

# ----------------------------------------------------------------------------
# The five workloads.  Sizes, dtypes and distributions follow the stated
# verify configurations; "N(0, s)" means standard deviation s.
# ----------------------------------------------------------------------------
CONFIGS = {
    "toy": dict(index=0, B=1, tree=("toy",), Hq=4, Hkv=4, D=64, L=128,
                dtype="f32", V=1000, p_sigma=2.0, q_sigma=0.5,
                kv_layout="contig"),
    "chain8": dict(index=1, B=1, tree=("chain", 8), Hq=32, Hkv=32, D=128,
                   L=2048, dtype="bf16", V=32000, p_sigma=3.0, q_sigma=1.0,
                   kv_layout="contig"),
    "medusa": dict(index=2, B=1, tree=("cartesian", (3, 5, 7)), Hq=32,
                   Hkv=32, D=128, L=4096, dtype="bf16", V=32000, p_sigma=3.0,
                   q_sigma=(0.5, 1.0, 1.5), kv_layout="contig"),
    "specinfer": dict(index=3, B=8, tree=("kschedule", (3, 2, 2, 1, 1)),
                      Hq=64, Hkv=8, D=128, L=8192, dtype="bf16", V=128256,
                      p_sigma=3.0, q_sigma=1.0, kv_layout="contig"),
    # Not one of the five: a lookahead-decoding pass (survey page, 8.2.3) with
    # W=5, N=4, G=5 -- "0" + 14 lookahead rows + 15 verify rows = 30 rows whose
    # attention mask is not a tree mask; shaped like chain8's layer.
    "lookahead": dict(index=5, B=1, tree=("chain", 29), Hq=32, Hkv=32, D=128, L=2048,
                      dtype="bf16", V=32000, p_sigma=3.0, q_sigma=1.0, kv_layout="contig",
                      visibility=("lookahead", 5, 4, 5)),
    "dynamic": dict(index=4, B=64, tree=("eagle2", 5, 8), kmax_per_req=16,
                    Hq=32, Hkv=8, D=128, L=("uniform", 512, 16384),
                    dtype="bf16", V=128256, p_sigma=3.0, q_sigma=1.0,
                    kv_layout="paged"),
}
CONFIG_ORDER = ["toy", "chain8", "medusa", "specinfer", "dynamic"]
BLOCK = 16


def _seed(*parts) -> int:
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    V: int
    dtype: str                 # "bf16" or "f32": Q/K/V element type
    kv_layout: str             # "contig" or "paged"
    parents: np.ndarray        # int32 [R], parent in local row numbers, -1 at roots
    row_offsets: np.ndarray    # int32 [B+1]
    prefix_len: np.ndarray     # int32 [B]
    tokens: np.ndarray         # int32 [R]; root rows hold the last accepted token
    device: str
    q: torch.Tensor            # [R][Hq][D]
    k_new: torch.Tensor        # [R][Hkv][D]
    v_new: torch.Tensor        # [R][Hkv][D]
    k_cache: torch.Tensor      # contig [B][Hkv][cap][D] | paged [nblk][Hkv][16][D]
    v_cache: torch.Tensor
    capacity: int              # contig only
    block_table: torch.Tensor | None   # int32 [B][max_blocks] (paged)
    p_logits: torch.Tensor     # float32 [R][V]
    q_logits: torch.Tensor     # float32 [R][V]; leaf rows are NaN (never needed)
    nonleaf: np.ndarray        # bool [R]
    seed: int = 0              # Philox key for the acceptance uniforms
    step: int = 0
    temperature: float = 1.0
    # per request: visibility of the new rows when the attention mask is not
    # the tree's ancestor mask (bool [n][n]); None for tree masks
    visibility: list | None = None
    block_size: int = BLOCK

    @property
    def R(self) -> int:
        return int(self.row_offsets[-1])

    def rows(self, b: int) -> int:
        return int(self.row_offsets[b + 1] - self.row_offsets[b])

    @property
    def max_rows(self) -> int:
        return int(np.diff(self.row_offsets).max())

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    # -- host views for CPU-side consumers --------------------------------
    def prefix_kv(self, b: int):
        """float64 numpy (K, V), each [Hkv][L_b][D], for request b's prefix."""
        L = int(self.prefix_len[b])
        if self.kv_layout == "contig":
            k = self.k_cache[b, :, :L]
            v = self.v_cache[b, :, :L]
        else:
            nb = (L + self.block_size - 1) // self.block_size
            ids = self.block_table[b, :nb].long()
            k = self.k_cache[ids].permute(1, 0, 2, 3).reshape(self.Hkv, -1, self.D)[:, :L]
            v = self.v_cache[ids].permute(1, 0, 2, 3).reshape(self.Hkv, -1, self.D)[:, :L]
        return (k.detach().to("cpu", torch.float64).numpy(),
                v.detach().to("cpu", torch.float64).numpy())

    def host(self, name: str) -> np.ndarray:
        t = getattr(self, name)
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.detach().to("cpu").double().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def _tree_for(cfg, rng, B):
    kind = cfg["tree"][0]
    if kind == "toy":
        return [trees.toy_tree() for _ in range(B)]
    if kind == "chain":
        return [trees.chain(cfg["tree"][1]) for _ in range(B)]
    if kind == "cartesian":
        return [trees.cartesian(cfg["tree"][1]) for _ in range(B)]
    if kind == "kschedule":
        return [trees.k_schedule(cfg["tree"][1]) for _ in range(B)]
    if kind == "given":                 # trees supplied by the caller (e.g. a tree builder)
        return [np.asarray(t, dtype=np.int32) for t in cfg["tree"][1]]
    if kind == "eagle2":
        topk, max_depth = cfg["tree"][1], cfg["tree"][2]
        sizes = trees.echo_budget(rng, B, cfg.get("kmax_per_req", 16) * B)
        return [trees.eagle2_tree(rng, int(n), topk, max_depth) for n in sizes]
    raise ValueError(kind)


def prefix_lengths(name: str, **over) -> np.ndarray:
    """The prefix lengths ``make(name, **over)`` draws, without building the
    tensors (same seed, same order of draws)."""
    cfg = dict(CONFIGS[name])
    for k in ("seed", "step", "temperature"):
        over.pop(k, None)
    tag = over.pop("tag", 0)
    cfg.update(over)
    base = (1000 + cfg["index"], tag, tuple(sorted((k, repr(v)) for k, v in over.items())))
    rng = np.random.default_rng(_seed(*base, "host"))
    B = cfg["B"]
    _tree_for(cfg, rng, B)
    Lspec = cfg["L"]
    if isinstance(Lspec, tuple):
        return rng.integers(Lspec[1], Lspec[2], size=B, endpoint=True).astype(np.int32)
    if isinstance(Lspec, (list, np.ndarray)):
        return np.asarray(Lspec, dtype=np.int32)
    return np.full(B, int(Lspec), dtype=np.int32)


def make(name: str, device: str = "cpu", **over) -> Workload:
    """Build workload ``name`` (one of CONFIGS) on ``device``.

    ``over`` replaces any config field (B, L, V, Hq, Hkv, D, kv_layout, tree,
    p_sigma, q_sigma ...) to get reduced-size variants with the same recipe;
    ``seed``/``step``/``temperature`` set the acceptance parameters.
    """
    cfg = dict(CONFIGS[name])
    seed = over.pop("seed", 0)
    step = over.pop("step", 0)
    temperature = over.pop("temperature", 1.0)
    tag = over.pop("tag", 0)
    cfg.update(over)
    base = (1000 + cfg["index"], tag, tuple(sorted((k, repr(v)) for k, v in over.items())))
    rng = np.random.default_rng(_seed(*base, "host"))

    B, Hq, Hkv, D, V = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["V"]
    tlist = _tree_for(cfg, rng, B)
    sizes = np.array([len(t) for t in tlist], dtype=np.int32)
    row_offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    parents = np.concatenate(tlist).astype(np.int32)
    R = int(row_offsets[-1])

    Lspec = cfg["L"]
    if isinstance(Lspec, tuple):
        prefix_len = rng.integers(Lspec[1], Lspec[2], size=B, endpoint=True).astype(np.int32)
    elif isinstance(Lspec, (list, np.ndarray)):
        prefix_len = np.asarray(Lspec, dtype=np.int32)
    else:
        prefix_len = np.full(B, int(Lspec), dtype=np.int32)

    nonleaf = np.zeros(R, dtype=bool)
    depth = np.zeros(R, dtype=np.int32)
    for b in range(B):
        o = row_offsets[b]
        for i in range(1, sizes[b]):
            nonleaf[o + parents[o + i]] = True
            depth[o + i] = depth[o + parents[o + i]] + 1

    tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32

    def normal(shape, *tagp, scale=1.0):
        g = _gen(device, *base, *tagp)
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        return x

    q = normal((R, Hq, D), "q").to(tdt)
    k_new = normal((R, Hkv, D), "knew").to(tdt)
    v_new = normal((R, Hkv, D), "vnew").to(tdt)

    block_table = None
    layout = cfg["kv_layout"]
    need = prefix_len.astype(np.int64) + sizes
    if layout == "contig":
        capacity = int(((need.max() + BLOCK - 1) // BLOCK) * BLOCK)
        k_cache = torch.empty((B, Hkv, capacity, D), dtype=tdt, device=device)
        v_cache = torch.empty_like(k_cache)
        for b in range(B):
            L = int(prefix_len[b])
            k_cache[b, :, :L] = normal((Hkv, L, D), "kc", b).to(tdt)
            v_cache[b, :, :L] = normal((Hkv, L, D), "vc", b).to(tdt)
            # slots past the prefix hold junk until the tree rows are appended
            k_cache[b, :, L:] = float("nan")
            v_cache[b, :, L:] = float("nan")
    else:
        capacity = 0
        nblocks_req = (need + BLOCK - 1) // BLOCK
        nblk = int(nblocks_req.sum()) + 8
        perm = rng.permutation(nblk).astype(np.int32)
        mbps = int(nblocks_req.max())
        bt = np.full((B, mbps), -1, dtype=np.int32)
        pos = 0
        for b in range(B):
            nb = int(nblocks_req[b])
            bt[b, :nb] = perm[pos:pos + nb]
            pos += nb
        block_table = torch.from_numpy(bt).to(device)
        k_cache = normal((nblk, Hkv, BLOCK, D), "kc").to(tdt)
        v_cache = normal((nblk, Hkv, BLOCK, D), "vc").to(tdt)

    p_logits = normal((R, V), "p", scale=float(cfg["p_sigma"]))
    qs = cfg["q_sigma"]
    noise = normal((R, V), "qn")
    if isinstance(qs, tuple):
        sig = torch.tensor([qs[min(int(d), len(qs) - 1)] for d in depth],
                           dtype=torch.float32, device=device)
        q_logits = p_logits + noise * sig[:, None]
    else:
        q_logits = p_logits + noise * float(qs)
    del noise
    leaf_rows = torch.from_numpy(np.nonzero(~nonleaf)[0]).to(device)
    q_logits[leaf_rows] = float("nan")

    # Draft tokens: child c of u ~ softmax(q_logits[u]) by Gumbel-max.
    tokens = np.zeros(R, dtype=np.int32)
    g_tok = _gen(device, *base, "tok")
    child_rows = np.array([row_offsets[b] + i for b in range(B) for i in range(1, sizes[b])],
                          dtype=np.int64)
    par_rows = np.array([row_offsets[b] + parents[row_offsets[b] + i] for b in range(B)
                         for i in range(1, sizes[b])], dtype=np.int64)
    CH = 256
    for s in range(0, len(child_rows), CH):
        pr = torch.from_numpy(par_rows[s:s + CH]).to(device)
        u = torch.rand((len(pr), V), generator=g_tok, device=device, dtype=torch.float64)
        u.clamp_(min=1e-300)
        gum = -torch.log(-torch.log(u))
        pick = torch.argmax(q_logits[pr].double() + gum, dim=1)
        tokens[child_rows[s:s + CH]] = pick.cpu().numpy().astype(np.int32)
    root_rows = row_offsets[:-1]
    tokens[root_rows] = rng.integers(0, V, size=B)
    if cfg.get("given_tokens") is not None:      # the tree builder's tokens
        tokens = np.asarray(cfg["given_tokens"], dtype=np.int32).copy()
        assert tokens.shape == (R,)
    if cfg.get("draft", "sample") == "topk":
        kids = {}
        for c, u in zip(child_rows, par_rows):
            kids.setdefault(int(u), []).append(int(c))
        us = sorted(kids)
        kmax = max(len(v) for v in kids.values())
        for s in range(0, len(us), CH):
            blk = us[s:s + CH]
            order = torch.sort(q_logits[torch.tensor(blk, device=device)], dim=1,
                               descending=True, stable=True).indices[:, :kmax].cpu().numpy()
            for j, u in enumerate(blk):
                for i, c in enumerate(kids[u]):
                    tokens[c] = int(order[j, i])

    visibility = None
    if cfg.get("visibility") is not None:
        kind, *args = cfg["visibility"]
        assert kind == "lookahead"
        visibility = [masks.lookahead_visibility(*args) for _ in range(B)]
        assert all(v.shape[0] == sizes[b] for b, v in enumerate(visibility))
    return Workload(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, V=V, dtype=cfg["dtype"],
                    kv_layout=layout, parents=parents, row_offsets=row_offsets,
                    prefix_len=prefix_len, tokens=tokens, device=device, q=q,
                    k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                    capacity=capacity, block_table=block_table, p_logits=p_logits,
                    q_logits=q_logits, nonleaf=nonleaf, seed=seed, step=step,
                    temperature=temperature, visibility=visibility)
