"""Seeded synthetic inputs for the batched verify step.

This module only draws random numbers and lays them out; it holds none of the
verify step's arithmetic (no softmax, no accept test, no residual, no CDF).
Both the GPU library's tests / benchmark and the fp64 oracle are fed from it.

Five workloads, named by what they are:

  tiny      B=1,   K=4, V=1000,   fp32, T=1.0  target N(0,2^2); draft = target + N(0,1)
  peaked    B=8,   K=4, V=32000,  bf16, T=1.0  target N(0,3^2) + 8 on 20 ids/row;
                                               draft = target + N(0,1.5^2)
  headline  B=64,  K=5, V=128256, bf16, T=0.8  target as "peaked"; draft noise std
                                               per request ~ U(0.5, 3.0)
  greedy    B=256, K=3, V=151936, bf16         target N(0,2^2) + 10 on one id/row;
                                               draft = target argmax w.p. 0.7 else a
                                               uniform id (one-hot drafts)
  ragged    B=512, K=8, V=151936, fp32, T=0.6  target N(0,2.5^2) - 1.1 ln(rank),
                                               rank = 1 + pi(t) for one seeded
                                               permutation pi shared by all rows;
                                               draft = target + N(0,1); k_b ~ U{1..8}

Generation recipe:
  * numpy Generator(Philox); the seed of workload c is 1000 + c;
    SeedSequence([seed, set_index]).spawn(4) gives four streams:
    logits / noise / drafts / uniforms.
  * logits are drawn in fp64, cast to fp32, then to bf16 with
    round-to-nearest-even where the workload is bf16 (kept as uint16 bits).
  * draft tokens are drawn from the *stored* draft logits at temperature T
    with the Gumbel-max trick (argmax of d/T + Gumbel noise), so the q the
    verifier sees is the q that drew them.
  * uniforms are fp32 in [0, 1) (multiples of 2^-24).
  * padded rows of the ragged workload (target rows i > k_b, draft rows
    i >= k_b) are filled with NaN: a verifier that reads them is wrong.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

NAMES = ("tiny", "peaked", "headline", "greedy", "ragged")

SHAPES = {
    "tiny": dict(B=1, K=4, V=1000, dtype="fp32", T=1.0, greedy=False),
    "peaked": dict(B=8, K=4, V=32000, dtype="bf16", T=1.0, greedy=False),
    "headline": dict(B=64, K=5, V=128256, dtype="bf16", T=0.8, greedy=False),
    "greedy": dict(B=256, K=3, V=151936, dtype="bf16", T=1.0, greedy=True),
    "ragged": dict(B=512, K=8, V=151936, dtype="fp32", T=0.6, greedy=False),
}


@dataclass
class Workload:
    name: str
    B: int
    K: int
    V: int
    dtype: str                      # "fp32" or "bf16"
    temperature: float
    greedy: bool
    target: np.ndarray              # [B, K+1, V] float32 or uint16 (bf16 bits)
    draft: Optional[np.ndarray]     # [B, K, V] like target, or None (one-hot drafts)
    draft_tokens: np.ndarray        # [B, K] int32
    uniforms: np.ndarray            # [B, K+1] float32 in [0, 1)
    k_per_req: Optional[np.ndarray] = None   # [B] int32 or None (all K)
    meta: dict = field(default_factory=dict)

    def k_of(self, b: int) -> int:
        return int(self.K if self.k_per_req is None else self.k_per_req[b])

    def verified_positions(self) -> int:
        """Sum over requests of (k_b + 1): the positions one step verifies."""
        if self.k_per_req is None:
            return self.B * (self.K + 1)
        return int(np.sum(self.k_per_req.astype(np.int64) + 1))


def _rngs(seed: int, set_index: int):
    ss = np.random.SeedSequence([seed, set_index])
    return [np.random.Generator(np.random.Philox(s)) for s in ss.spawn(4)]


def bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns with round-to-nearest-even (finite inputs;
    NaN stays NaN)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_as_f32(a: np.ndarray) -> np.ndarray:
    """The stored logits (fp32 array or bf16 bits) as float32 values."""
    return bf16_to_f32(a) if a.dtype == np.uint16 else a


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    f = x64.astype(np.float32)
    return bf16_bits(f) if dtype == "bf16" else f


def gumbel_draw(logits_f32: np.ndarray, temperature: float, rng) -> np.ndarray:
    """Draw one token id per row with probability proportional to
    exp(logit / T) via the Gumbel-max trick: argmax_t (l_t / T + G_t).
    This is the drafter's side of the workload, not the verifier."""
    rows = logits_f32.reshape(-1, logits_f32.shape[-1])
    out = np.empty(rows.shape[0], np.int32)
    inv_t = 1.0 / float(temperature)
    for r in range(rows.shape[0]):
        g = rng.gumbel(size=rows.shape[1])
        out[r] = int(np.argmax(rows[r].astype(np.float64) * inv_t + g))
    return out.reshape(logits_f32.shape[:-1])


def _peaked_target(rng, B, R, V, std, boost, n_peaks):
    x = rng.standard_normal((B, R, V)) * std
    for b in range(B):
        for i in range(R):
            ids = rng.choice(V, size=n_peaks, replace=False)
            x[b, i, ids] += boost
    return x


def make(name: str, set_index: int = 0, B: Optional[int] = None, V: Optional[int] = None,
         K: Optional[int] = None) -> Workload:
    """Build one seeded input set of a named workload.

    B, V and K may be overridden to get the same recipe at a smaller (or
    ragged) size for tests; the defaults are the full sizes.
    """
    if name not in SHAPES:
        raise KeyError(name)
    cfg = dict(SHAPES[name])
    if B is not None:
        cfg["B"] = B
    if V is not None:
        cfg["V"] = V
    if K is not None:
        cfg["K"] = K
    B, K, V, dt, T = cfg["B"], cfg["K"], cfg["V"], cfg["dtype"], cfg["T"]
    seed = 1000 + NAMES.index(name)
    r_logit, r_noise, r_draft, r_unif = _rngs(seed, set_index)
    k_per_req = None
    meta = {"seed": seed, "set_index": set_index}

    if name == "tiny":
        l = r_logit.standard_normal((B, K + 1, V)) * 2.0
        d = l[:, :K, :] + r_noise.standard_normal((B, K, V))
    elif name == "peaked":
        l = _peaked_target(r_logit, B, K + 1, V, 3.0, 8.0, min(20, V))
        d = l[:, :K, :] + r_noise.standard_normal((B, K, V)) * 1.5
    elif name == "headline":
        l = _peaked_target(r_logit, B, K + 1, V, 3.0, 8.0, min(20, V))
        sig = r_noise.uniform(0.5, 3.0, size=B)
        meta["draft_noise_std"] = sig
        d = l[:, :K, :] + r_noise.standard_normal((B, K, V)) * sig[:, None, None]
    elif name == "greedy":
        l = r_logit.standard_normal((B, K + 1, V)) * 2.0
        peak = r_logit.integers(0, V, size=(B, K + 1))
        np.add.at(l, (np.arange(B)[:, None], np.arange(K + 1)[None, :], peak), 10.0)
        d = None
    elif name == "ragged":
        k_per_req = r_draft.integers(1, K + 1, size=B).astype(np.int32)
        perm = r_logit.permutation(V)
        offset = -1.1 * np.log(1.0 + perm.astype(np.float64))
        # Stored per request to keep host memory at the fp32 size.
        l = None
        d = None
        t32 = np.full((B, K + 1, V), np.nan, np.float32)
        d32 = np.full((B, K, V), np.nan, np.float32)
        for b in range(B):
            kb = int(k_per_req[b])
            lb = r_logit.standard_normal((kb + 1, V)) * 2.5 + offset
            t32[b, :kb + 1] = lb
            d32[b, :kb] = lb[:kb] + r_noise.standard_normal((kb, V))
        meta["stored"] = (t32, d32)
    else:  # pragma: no cover
        raise KeyError(name)

    if "stored" in meta:
        target, draft = meta.pop("stored")
    else:
        target = _store(l, dt)
        draft = None if d is None else _store(d, dt)
    del l, d

    if name == "greedy":
        # Deterministic (n-gram style) drafts: the target argmax of the stored
        # row with probability 0.7, otherwise a uniformly random id.
        vals = stored_as_f32(target)[:, :K, :]
        am = np.argmax(vals, axis=-1).astype(np.int32)
        hit = r_draft.random((B, K)) < 0.7
        rnd = r_draft.integers(0, V, size=(B, K)).astype(np.int32)
        tokens = np.where(hit, am, rnd).astype(np.int32)
    else:
        tokens = np.zeros((B, K), np.int32)
        dv = stored_as_f32(draft)
        for b in range(B):
            kb = K if k_per_req is None else int(k_per_req[b])
            if kb > 0:
                tokens[b, :kb] = gumbel_draw(dv[b, :kb], T, r_draft)
    uniforms = r_unif.random((B, K + 1), dtype=np.float32)
    return Workload(name=name, B=B, K=K, V=V, dtype=dt, temperature=T, greedy=cfg["greedy"],
                    target=target, draft=draft, draft_tokens=tokens, uniforms=uniforms,
                    k_per_req=k_per_req, meta=meta)


def near_drafts(sigma: float, dtype: str = "bf16", B: int = 1024, distinct: int = 32,
                V: int = 128256, K: int = 1, set_index: int = 0,
                force_reject: bool = True) -> Workload:
    """The high-acceptance regime: a draft distribution close to the target
    one, as a good drafter gives ("Speculative Decoding from First
    Principles", "What the numbers say": most first drafts accepted).

    `distinct` peaked target row blocks (N(0, 3^2) + 8 on 20 ids per row,
    the headline recipe, T = 0.8) with draft rows = target + N(0, sigma^2),
    each block repeated over B / distinct requests; every request draws its
    own drafted tokens from the stored draft rows (Gumbel-max at T) and its
    own uniforms.  With force_reject the accept uniforms are 1 - 2^-18, so a
    draft is rejected whenever p(x)/q(x) < 1 - 2^-18 -- about half of the
    requests -- while an accepted draft (ratio 1) stays 3.8e-6 away from its
    threshold; the final uniform sweeps [0, 1) over the requests that share
    a block.
    Seed 1008; the stream set is SeedSequence([1008, set_index, round(sigma
    * 1e6), dtype])."""
    if B % distinct:
        raise ValueError("B must be a multiple of distinct")
    T = 0.8
    ss = np.random.SeedSequence([1008, set_index, int(round(sigma * 1e6)), 1 if dtype == "bf16" else 0])
    r_logit, r_noise, r_draft, r_unif = [np.random.Generator(np.random.Philox(s)) for s in ss.spawn(4)]
    l = _peaked_target(r_logit, distinct, K + 1, V, 3.0, 8.0, min(20, V))
    d = l[:, :K, :] + r_noise.standard_normal((distinct, K, V)) * sigma
    t_blk, d_blk = _store(l, dtype), _store(d, dtype)
    del l, d
    rep = B // distinct
    target = np.ascontiguousarray(np.repeat(t_blk, rep, axis=0))
    draft = np.ascontiguousarray(np.repeat(d_blk, rep, axis=0))
    dv = stored_as_f32(d_blk)
    tokens = np.empty((B, K), np.int32)
    inv_t = 1.0 / T
    for g in range(distinct):
        for i in range(K):
            gum = r_draft.gumbel(size=(rep, V))
            tokens[g * rep:(g + 1) * rep, i] = np.argmax(dv[g, i].astype(np.float64) * inv_t + gum, axis=-1)
    uniforms = r_unif.random((B, K + 1), dtype=np.float32)
    if force_reject:
        uniforms[:, :K] = np.float32(1.0 - 2.0 ** -18)
    return Workload(name="near", B=B, K=K, V=V, dtype=dtype, temperature=T, greedy=False,
                    target=target, draft=draft, draft_tokens=tokens, uniforms=uniforms,
                    meta={"seed": 1008, "set_index": set_index, "sigma": sigma,
                          "distinct": distinct})


def tiny_steps(n_steps: int, set_index: int = 0) -> Workload:
    """The tiny workload run for many steps: the logits stay fixed and every
    step draws fresh drafts and uniforms.  The steps are laid out as a batch
    of n_steps independent requests that share the same logit rows."""
    base = make("tiny", set_index=set_index)
    K, V = base.K, base.V
    rng_d, rng_u = [np.random.Generator(np.random.Philox(s))
                    for s in np.random.SeedSequence([base.meta["seed"], set_index, 7]).spawn(2)]
    target = np.ascontiguousarray(np.broadcast_to(base.target[0], (n_steps, K + 1, V)))
    draft = np.ascontiguousarray(np.broadcast_to(base.draft[0], (n_steps, K, V)))
    # All steps share the rows, so draw each position's drafts in one batch.
    tokens = np.empty((n_steps, K), np.int32)
    inv_t = 1.0 / base.temperature
    for i in range(K):
        g = rng_d.gumbel(size=(n_steps, V))
        tokens[:, i] = np.argmax(base.draft[0, i].astype(np.float64) * inv_t + g, axis=-1)
    uniforms = rng_u.random((n_steps, K + 1), dtype=np.float32)
    return Workload(name="tiny", B=n_steps, K=K, V=V, dtype=base.dtype,
                    temperature=base.temperature, greedy=False, target=target, draft=draft,
                    draft_tokens=tokens, uniforms=uniforms, meta=dict(base.meta, steps=n_steps))


def ngram_contexts(B: int = 256, L_max: int = 4096, V: int = 151936, set_index: int = 0,
                   copy_prob: float = 0.6):
    """Copy-heavy token contexts for the n-gram drafter (a stand-in for the
    code-edit / RAG traffic the pages name, where the output quotes its
    input): each request's context is built from spans of 8..64 tokens,
    each span either copied from a random earlier position of the same
    context (probability copy_prob) or drawn uniformly from [0, V).
    Lengths are uniform on [L_max / 4, L_max].  Returns (context [B, L_max]
    int32, padded with uniform ids past each length; context_len [B] int32).
    Seed 1006, stream set_index."""
    rng = np.random.default_rng(np.random.SeedSequence([1006, set_index]))
    ctx = rng.integers(0, V, size=(B, L_max), dtype=np.int64).astype(np.int32)
    lens = rng.integers(max(1, L_max // 4), L_max + 1, size=B).astype(np.int32)
    for b in range(B):
        L = int(lens[b])
        pos = min(L, 64)
        while pos < L:
            m = int(rng.integers(8, 65))
            m = min(m, L - pos)
            if rng.random() < copy_prob:
                src = int(rng.integers(0, pos))
                if src + m <= pos:
                    ctx[b, pos:pos + m] = ctx[b, src:src + m]
                else:                # overlaps the span being written
                    for i in range(m):
                        ctx[b, pos + i] = ctx[b, src + i]
            pos += m
    return ctx, lens


def tree_parents(branching) -> np.ndarray:
    """Parent links of a static draft tree flattened breadth first, the
    order of the pages' example [a, b, a1, a2, b1, b2]: branching[d] children
    under every node of depth d (the root has depth 0); -1 = the root."""
    parents, level = [], [-1]
    for m in branching:
        nxt = []
        for p in level:
            for _ in range(int(m)):
                parents.append(p)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.array(parents, np.int32)


@dataclass
class TreeWorkload:
    name: str
    B: int
    N: int
    V: int
    dtype: str
    target: np.ndarray              # [B, N+1, V]: row 0 after the root, row i+1 after node i
    node_tokens: np.ndarray         # [B, N] int32
    parents: np.ndarray             # [B, N] int32
    n_nodes: Optional[np.ndarray]   # [B] int32 or None (all N)
    meta: dict = field(default_factory=dict)

    def rows_read(self) -> int:
        nn = np.full(self.B, self.N) if self.n_nodes is None else self.n_nodes
        return int(np.sum(nn.astype(np.int64) + 1))


def tree(B: int = 64, V: int = 128256, branching=(3, 2, 2), set_index: int = 0,
         dtype: str = "bf16", hit: float = 0.7) -> TreeWorkload:
    """A batch of draft trees scored by one target pass: every request uses
    the static tree of `branching` (default 3 candidates at depth 1, 2 under
    each at depths 2 and 3: 21 nodes), target rows as the greedy workload's
    (N(0, 2^2) + 10 on one id per row).  The first child under each node --
    the draft's top candidate -- is the target argmax of the parent's stored
    row with probability `hit`, otherwise a uniform id; the other children
    (lower-ranked candidates) are uniform ids.  Seed 1007."""
    par1 = tree_parents(branching)
    N = len(par1)
    r_logit, r_noise, r_draft, _ = _rngs(1007, set_index)
    l = r_logit.standard_normal((B, N + 1, V)) * 2.0
    peak = r_logit.integers(0, V, size=(B, N + 1))
    np.add.at(l, (np.arange(B)[:, None], np.arange(N + 1)[None, :], peak), 10.0)
    target = _store(l, dtype)
    del l
    am = np.argmax(stored_as_f32(target), axis=-1).astype(np.int32)
    first = np.array([i == 0 or par1[i - 1] != par1[i] for i in range(N)], bool)
    parents = np.tile(par1, (B, 1))
    above = am[:, par1 + 1]                                  # argmax of each node's parent row
    take = first[None, :] & (r_draft.random((B, N)) < hit)
    rnd = r_draft.integers(0, V, size=(B, N)).astype(np.int32)
    tokens = np.where(take, above, rnd).astype(np.int32)
    return TreeWorkload(name="tree", B=B, N=N, V=V, dtype=dtype, target=target,
                        node_tokens=tokens, parents=parents.astype(np.int32), n_nodes=None,
                        meta={"seed": 1007, "set_index": set_index,
                              "branching": tuple(int(m) for m in branching)})
