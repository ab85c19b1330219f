"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
five seeded workloads at full size, on ragged and misaligned shapes, and on
the degenerate cases of the method."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_verification_10_amd import workloads
from tests.gpu_util import (seeded_sets, assert_workspace_clean, compare_verify, dev_logits,
                            oracle_verify, run_verify)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_decoding_verification_10_amd as sd
    sd.load(build_if_missing=False)


# ---------------------------------------------------------------------------
# Row statistics
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "peaked", "headline", "greedy", "ragged"])
def test_softmax_stats_full_size(name):
    import speculative_decoding_verification_10_amd as sd
    say("stats", name)
    wl = workloads.make(name)
    rows = wl.target.reshape(-1, wl.V)
    if name == "ragged":           # the NaN padding rows are not valid logits
        keep = np.concatenate([np.arange(wl.k_of(b) + 1) + b * (wl.K + 1) for b in range(wl.B)])
        rows = np.ascontiguousarray(rows[keep[:600]])
    T = wl.temperature
    m, z = sd.softmax_stats(dev_logits(rows), T)
    torch.cuda.synchronize()
    om, oz = oracle.softmax_stats(rows, T)
    assert np.array_equal(m.cpu().numpy().astype(np.float64), om)
    np.testing.assert_allclose(z.cpu().numpy().astype(np.float64), oz, rtol=1e-5)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V", [1, 7, 777, 1001, 4096, 20000, 65543])
def test_softmax_stats_ragged(dtype, V):
    import speculative_decoding_verification_10_amd as sd
    rng = np.random.default_rng(V)
    x = (rng.standard_normal((5, V)) * 3).astype(np.float32)
    if V > 1:
        x[1, : V // 2] = -np.inf
    arr = workloads.bf16_bits(x) if dtype == "bf16" else x
    for T in (1.0, 0.37):
        m, z = sd.softmax_stats(dev_logits(arr), T)
        torch.cuda.synchronize()
        om, oz = oracle.softmax_stats(arr, T)
        assert np.array_equal(m.cpu().numpy().astype(np.float64), om)
        np.testing.assert_allclose(z.cpu().numpy().astype(np.float64), oz, rtol=1e-5)


# ---------------------------------------------------------------------------
# Stochastic verify
# ---------------------------------------------------------------------------

# (config, flagged, differing, requests) of the stochastic full-size runs
# of the configs; test_verify_configs_mismatch_share holds their sum to the
# 0.01% bar.
_CONFIG_TALLY = []


def test_verify_tiny_10000_steps():
    say("verify tiny x10000")
    wl = workloads.tiny_steps(10_000)
    gpu = run_verify(wl)
    ref = oracle_verify(wl)
    nf, nd = compare_verify("tiny", gpu, ref)
    say("counts tiny steps 10000 requests", wl.B, "flagged", nf, "differ", nd)
    _CONFIG_TALLY.append(("tiny", nf, nd, wl.B))
    assert nd <= 1 + 0.1 * nf, (nd, nf)


@pytest.mark.parametrize("name,sets", [("peaked", 1000), ("headline", 20)])
def test_verify_full_size(name, sets):
    """Distinct seeded sets (set_index 0..sets-1): 1,000 steps of the peaked
    batch, 20 of the headline batch."""
    flagged = differ = total = 0
    for s, wl, ref in seeded_sets(name, sets, ahead=16 if name == "peaked" else 4):
        if s % 50 == 0 or name != "peaked":
            say("verify", name, "set", s)
        nf, nd = compare_verify("%s/%d" % (name, s), run_verify(wl), ref)
        flagged += nf
        differ += nd
        total += wl.B
    say("counts", name, "sets", sets, "requests", total, "flagged", flagged, "differ", differ)
    _CONFIG_TALLY.append((name, flagged, differ, total))
    # Every differing request is flagged (compare_verify).  A flagged final
    # draw lies within 1e-6 of a CDF boundary -- on peaked rows, any draw
    # among the tail tokens, whose own masses are below 2e-6 of S -- and the
    # fp32 path places boundaries to ~1e-7 of S, so it may decide at most
    # about a tenth of the flagged requests the other way.
    assert differ <= 1 + 0.1 * flagged, (differ, flagged)


def test_verify_ragged_full_size():
    """Three distinct seeded sets of the ragged batch (B = 512, k_b from 1 to
    8, V = 151,936, fp32)."""
    flagged = differ = total = 0
    for s, wl, ref in seeded_sets("ragged", 3, workers=3, ahead=2):
        say("verify ragged set", s)
        nf, nd = compare_verify("ragged/%d" % s, run_verify(wl), ref)
        flagged += nf
        differ += nd
        total += wl.B
    say("counts ragged sets 3 requests", total, "flagged", flagged, "differ", differ)
    _CONFIG_TALLY.append(("ragged", flagged, differ, total))
    assert differ <= 1 + 0.1 * flagged, (differ, flagged)


def test_verify_configs_mismatch_share():
    """Over the stochastic full-size runs above (10,000 tiny steps, 1,000
    peaked, 20 headline, 3 ragged): the requests that differ from the oracle,
    every one of them flagged, are under 0.01% of the requests."""
    if not _CONFIG_TALLY:
        pytest.skip("no full-size run in this session")
    flagged = sum(t[1] for t in _CONFIG_TALLY)
    differ = sum(t[2] for t in _CONFIG_TALLY)
    total = sum(t[3] for t in _CONFIG_TALLY)
    say("counts configs", [t[0] for t in _CONFIG_TALLY], "requests", total, "flagged", flagged, "differ", differ)
    assert differ < 1e-4 * total, (differ, total)


@pytest.mark.parametrize("name,B,V,K", [
    ("peaked", 2, 4096, 255),     # the largest K; the final tiles take the decision
    ("headline", 2, 40000, 255),  # the largest K; the decision taken once per request
    ("ragged", 3, 40000, 60),     # ragged k_b, decision once per request
])
def test_verify_long_drafts(name, B, V, K):
    say("verify long drafts", name, B, V, K)
    wl = workloads.make(name, set_index=1, B=B, V=V, K=K)
    ref = oracle_verify(wl)
    nf, nd = compare_verify("%s-K%d" % (name, K), run_verify(wl), ref)
    say("flagged", nf, "differ", nd, "of", wl.B)
    assert nd == 0


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V", [5, 777, 1001, 8192, 40001])
@pytest.mark.parametrize("one_hot", [False, True])
def test_verify_ragged_vocab(dtype, V, one_hot):
    rng = np.random.default_rng(V + one_hot)
    B, K, T = 48, 3, 0.9
    lt = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    ld = (lt[:, :K] + rng.standard_normal((B, K, V)) * 0.7).astype(np.float32)
    if dtype == "bf16":
        lt, ld = workloads.bf16_bits(lt), workloads.bf16_bits(ld)
    vals = workloads.stored_as_f32(ld)
    toks = np.stack([workloads.gumbel_draw(vals[:, i], T, rng) for i in range(K)], axis=1)
    uni = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.Workload("adhoc", B, K, V, dtype, T, False, lt, None if one_hot else ld,
                            toks.astype(np.int32), uni)
    compare_verify("V=%d" % V, run_verify(wl), oracle_verify(wl))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("one_hot", [False, True])
def test_verify_large_vocab(dtype, one_hot):
    """A vocabulary of 300007 tokens: in fp32 more than 1024 slabs of 64
    vectors per row, so the search lanes read part of their slab sums back
    from the workspace instead of holding them."""
    rng = np.random.default_rng(300007 + one_hot)
    B, K, V, T = 8, 3, 300007, 0.8
    lt = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    ld = (lt[:, :K] + rng.standard_normal((B, K, V)) * 0.5).astype(np.float32)
    if dtype == "bf16":
        lt, ld = workloads.bf16_bits(lt), workloads.bf16_bits(ld)
    vals = workloads.stored_as_f32(ld)
    toks = np.stack([workloads.gumbel_draw(vals[:, i], T, rng) for i in range(K)], axis=1)
    uni = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.Workload("adhoc", B, K, V, dtype, T, False, lt, None if one_hot else ld,
                            toks.astype(np.int32), uni)
    nf, nd = compare_verify("V=%d" % V, run_verify(wl), oracle_verify(wl))
    assert nd == 0


def test_verify_timed_matches_and_records():
    """specdec_verify_timed gives the bits of specdec_verify and has the
    dispatches take the caller's events (row kernel start and end, call
    end)."""
    import speculative_decoding_verification_10_amd as sd
    from tests.gpu_util import to_device
    wl = workloads.make("peaked", set_index=1)
    d = to_device(wl)
    args = (d["target"], d["draft"], d["draft_tokens"], d["uniforms"], wl.temperature)
    ref = sd.verify(*args, accept_prob=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    got = sd.verify(*args, accept_prob=True, events=ev)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    rows_ms, call_ms = ev[0].elapsed_time(ev[1]), ev[0].elapsed_time(ev[2])
    assert 0.0 < rows_ms < call_ms < 100.0, (rows_ms, call_ms)
    # Partial event lists: only the given events are recorded.
    e2 = torch.cuda.Event(enable_timing=True)
    got2 = sd.verify(*args, accept_prob=True, events=(None, None, e2))
    e2.synchronize()
    assert torch.equal(got2[0], ref[0])


def test_verify_misaligned_pointers():
    """Rows that do not start on a 16-byte boundary take the element-wise
    load path."""
    import speculative_decoding_verification_10_amd as sd
    rng = np.random.default_rng(5)
    B, K, V, T = 16, 2, 3000, 1.0
    lt = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    ld = (lt[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    uni = rng.random((B, K + 1), dtype=np.float32)
    big_t = torch.zeros(lt.size + 1, dtype=torch.float32, device="cuda")
    big_t[1:] = torch.from_numpy(lt.ravel()).cuda()
    big_d = torch.zeros(ld.size + 1, dtype=torch.float32, device="cuda")
    big_d[1:] = torch.from_numpy(ld.ravel()).cuda()
    t = big_t[1:].view(B, K + 1, V)
    d = big_d[1:].view(B, K, V)
    assert t.data_ptr() % 16 != 0
    ws = sd.Workspace(sd._lib.verify_workspace_bytes(B, K, V, 0, False), "cuda")
    res = sd.verify(t, d, torch.from_numpy(toks).cuda(), torch.from_numpy(uni).cuda(), T,
                    accept_prob=True, workspace=ws)
    assert_workspace_clean(ws)
    ref = oracle.verify(lt, ld, toks, uni, T)
    compare_verify("misaligned", res, ref)


def test_verify_edge_cases():
    """K = 0 (plain sampling), k_b = 0 for some requests, q = p (all
    accepted), disjoint supports (first draft always rejected), -inf logits."""
    rng = np.random.default_rng(17)
    V, T = 300, 0.7
    # K = 0
    lt = (rng.standard_normal((9, 1, V)) * 2).astype(np.float32)
    uni = rng.random((9, 1), dtype=np.float32)
    wl = workloads.Workload("k0", 9, 0, V, "fp32", T, False, lt, None,
                            np.zeros((9, 0), np.int32), uni)
    compare_verify("K=0", run_verify(wl), oracle_verify(wl))
    # q = p and k_b = 0 mixed
    B, K = 20, 4
    lt = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    ld = lt[:, :K].copy()
    kp = rng.integers(0, K + 1, size=B).astype(np.int32)
    for b in range(B):
        lt[b, kp[b] + 1:] = np.nan
        ld[b, kp[b]:] = np.nan
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    uni = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.Workload("qp", B, K, V, "fp32", T, False, lt, ld, toks, uni, k_per_req=kp)
    gpu = run_verify(wl)
    ref = oracle_verify(wl)
    compare_verify("q=p", gpu, ref)
    assert np.array_equal(gpu[1].cpu().numpy(), kp)
    # disjoint supports with -inf
    lt = np.full((B, 2, V), -np.inf, np.float32)
    ld = np.full((B, 1, V), -np.inf, np.float32)
    lt[:, :, :100] = rng.standard_normal((B, 2, 100)).astype(np.float32)
    ld[:, :, 200:] = rng.standard_normal((B, 1, 100)).astype(np.float32)
    toks = rng.integers(200, V, size=(B, 1)).astype(np.int32)
    uni = rng.random((B, 2), dtype=np.float32)
    wl = workloads.Workload("disjoint", B, 1, V, "fp32", 1.0, False, lt, ld, toks, uni)
    gpu = run_verify(wl)
    compare_verify("disjoint", gpu, oracle_verify(wl))
    assert np.all(gpu[1].cpu().numpy() == 0)
    assert np.all(gpu[0].cpu().numpy()[:, 0] < 100)


def test_verify_deterministic_and_reusable_workspace():
    """Reruns give identical bits, reusing one workspace across calls of
    different shapes (it is left zeroed after every call)."""
    import speculative_decoding_verification_10_amd as sd
    from tests.gpu_util import to_device
    wl = workloads.make("peaked", set_index=3)
    small = workloads.make("peaked", set_index=4, B=3, V=5000)
    ws = sd.Workspace(sd._lib.verify_workspace_bytes(wl.B, wl.K, wl.V, 1, False), "cuda")

    def call(w):
        d = to_device(w)
        r = sd.verify(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], w.temperature,
                      accept_prob=True, workspace=ws)
        assert_workspace_clean(ws)
        return r

    a = call(wl)
    ref_small = oracle_verify(small)
    for _ in range(5):
        b = call(wl)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
        compare_verify("small", call(small), ref_small)


def test_verify_workspace_needs_no_initialisation():
    """A workspace full of random bytes (error word aside) gives the same
    results: every scratch word is set before it is read in the same call."""
    import speculative_decoding_verification_10_amd as sd
    from tests.gpu_util import to_device
    wl = workloads.make("peaked", set_index=2, B=6, V=9000)
    ref = oracle_verify(wl)
    ws = sd.Workspace(sd._lib.verify_workspace_bytes(wl.B, wl.K, wl.V, 1, False), "cuda")
    g = torch.Generator(device="cuda").manual_seed(11)
    for _ in range(3):
        ws.tensor.random_(0, 256, generator=g)
        ws.tensor[:4] = 0
        d = to_device(wl)
        res = sd.verify(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], wl.temperature,
                        accept_prob=True, workspace=ws)
        assert_workspace_clean(ws)
        nf, nd = compare_verify("garbage workspace", res, ref)
        assert nd == 0


def test_greedy_workspace_needs_no_initialisation():
    """Greedy on a workspace of random bytes (error word aside), shared with
    verify calls in between: the same results every time."""
    import speculative_decoding_verification_10_amd as sd
    from tests.gpu_util import to_device
    gw = workloads.make("greedy", set_index=2, B=12, V=9001)
    wl = workloads.make("peaked", set_index=3, B=4, V=9001)
    gref = oracle.verify_greedy(gw.target, gw.draft_tokens)
    code = 1 if gw.dtype == "bf16" else 0
    nb = max(int(sd._lib.load().specdec_verify_greedy_workspace_bytes(gw.B, gw.K, gw.V, code)),
             sd._lib.verify_workspace_bytes(wl.B, wl.K, wl.V, 1, False))
    ws = sd.Workspace(nb, "cuda")
    g = torch.Generator(device="cuda").manual_seed(5)
    t = dev_logits(gw.target)
    toks = torch.from_numpy(gw.draft_tokens).cuda()
    d = to_device(wl)
    for _ in range(3):
        ws.tensor.random_(0, 256, generator=g)
        ws.tensor[:4] = 0
        out, nacc, _ = sd.verify_greedy(t, toks, workspace=ws)
        assert_workspace_clean(ws)
        assert np.array_equal(out.cpu().numpy(), gref["out_tokens"])
        assert np.array_equal(nacc.cpu().numpy(), gref["num_accepted"])
        sd.verify(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], wl.temperature,
                  workspace=ws)


def test_default_workspaces_across_entry_points():
    """verify, softmax_stats and verify_greedy called in turn on one stream
    with the module's cached workspaces."""
    import speculative_decoding_verification_10_amd as sd
    from tests.gpu_util import to_device
    wl = workloads.make("peaked", set_index=0, B=5, V=7000)
    gw = workloads.make("greedy", set_index=0, B=7, V=7000)
    ref = oracle_verify(wl)
    gref = oracle.verify_greedy(gw.target, gw.draft_tokens)
    d = to_device(wl)
    t = dev_logits(gw.target)
    for _ in range(3):
        res = sd.verify(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], wl.temperature,
                        accept_prob=True)
        torch.cuda.synchronize()
        assert compare_verify("cached", res, ref)[1] == 0
        sd.softmax_stats(d["target"].view(-1, wl.V), wl.temperature)
        out, nacc, _ = sd.verify_greedy(t, torch.from_numpy(gw.draft_tokens).cuda())
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), gref["out_tokens"])
        assert np.array_equal(nacc.cpu().numpy(), gref["num_accepted"])


# ---------------------------------------------------------------------------
# Acceptance telemetry
# ---------------------------------------------------------------------------

def test_acceptance_counts_from_verify_outputs():
    """Counts from the GPU verify outputs of the ragged and headline
    workloads, accumulated over calls, equal the oracle's counts of the same
    outputs (and of the oracle's own outputs, up to flagged requests)."""
    import speculative_decoding_verification_10_amd as sd
    for name, kw in (("ragged", dict(B=100, V=5000)), ("headline", dict(B=16, V=20000))):
        wl = workloads.make(name, set_index=2, **kw)
        out, nacc, _ = run_verify(wl, accept_prob=False)
        kp = None if wl.k_per_req is None else torch.from_numpy(wl.k_per_req).cuda()
        cnt = sd.acceptance_counts(nacc, wl.K, kp)
        cnt = sd.acceptance_counts(nacc, wl.K, kp, cnt)
        torch.cuda.synchronize()
        n_host = nacc.cpu().numpy()
        ref = oracle.acceptance_counts(n_host, wl.K, wl.k_per_req)
        ref = oracle.acceptance_counts(n_host, wl.K, wl.k_per_req, ref)
        assert np.array_equal(cnt.cpu().numpy().astype(np.uint64), ref), name
        k, at, ad, sp = sd.choose_k(cnt, 0.05, 1, wl.K)
        assert (k, at, ad, sp) == oracle.choose_k(ref, 0.05, 1, wl.K)


@pytest.mark.parametrize("B,K", [(1, 1), (300, 255), (65535, 8), (257, 3)])
def test_acceptance_counts_random(B, K):
    """Random (n_b <= k_b <= K) over several workgroups (atomic adds of
    partial counts), bit-exact against the oracle."""
    import speculative_decoding_verification_10_amd as sd
    rng = np.random.default_rng(B * 1000 + K)
    kp = rng.integers(0, K + 1, size=B).astype(np.int32)
    n = (rng.random(B) * (kp + 1)).astype(np.int32)
    cnt = sd.acceptance_counts(torch.from_numpy(n).cuda(), K, torch.from_numpy(kp).cuda())
    torch.cuda.synchronize()
    ref = oracle.acceptance_counts(n, K, kp)
    assert np.array_equal(cnt.cpu().numpy().astype(np.uint64), ref)


# ---------------------------------------------------------------------------
# n-gram drafter
# ---------------------------------------------------------------------------

def _ngram_check(ctx, lens, n_min, n_max, K):
    import speculative_decoding_verification_10_amd as sd
    d, k = sd.ngram_propose(torch.from_numpy(ctx).cuda(), torch.from_numpy(lens).cuda(),
                            n_min, n_max, K)
    torch.cuda.synchronize()
    rd, rk = oracle.ngram_propose(ctx, lens, n_min, n_max, K)
    assert np.array_equal(k.cpu().numpy(), rk), (n_min, n_max, K)
    assert np.array_equal(d.cpu().numpy(), rd), (n_min, n_max, K)
    return rk


@pytest.mark.parametrize("n_min,n_max,K", [(1, 4, 3), (2, 5, 8), (1, 1, 1), (3, 64, 255)])
def test_ngram_copy_heavy_contexts(n_min, n_max, K):
    """The seeded copy-heavy contexts (256 requests, up to 4096 tokens),
    bit-exact against the oracle."""
    from speculative_decoding_verification_10_amd import workloads
    ctx, lens = workloads.ngram_contexts(set_index=n_max)
    rk = _ngram_check(ctx, lens, n_min, n_max, K)
    assert rk.max() > 0


def test_ngram_edge_cases():
    """Empty, one- and two-token contexts, constant runs (matches that run
    into the suffix), a vocabulary of two ids, padding past each length
    that must never be read, and a 200,000-token context."""
    rng = np.random.default_rng(3)
    B, Ls = 40, 300
    ctx = rng.integers(0, 3, size=(B, Ls)).astype(np.int32)
    lens = np.array([0, 1, 2, 3] + list(rng.integers(0, Ls + 1, size=B - 4)), np.int32)
    ctx[5, :] = 7                      # a constant run
    lens[5] = 100
    ctx[6, :] = rng.integers(0, 2, size=Ls)
    for b in range(B):                 # padding: ids that never occur in the contexts
        ctx[b, lens[b]:] = 1000 + b
    for n_min, n_max, K in [(1, 4, 5), (1, 64, 255), (2, 2, 1)]:
        _ngram_check(ctx, lens, n_min, n_max, K)
    long = rng.integers(0, 50, size=(2, 200000)).astype(np.int32)
    long[1, -40:] = long[1, 1000:1040]
    _ngram_check(long, np.array([200000, 200000], np.int32), 1, 8, 16)


# ---------------------------------------------------------------------------
# Greedy verify
# ---------------------------------------------------------------------------

def _greedy(wl, kp=None):
    import speculative_decoding_verification_10_amd as sd
    t = dev_logits(wl.target)
    code = 1 if wl.dtype == "bf16" else 0
    ws = sd.Workspace(int(sd._lib.load().specdec_verify_greedy_workspace_bytes(wl.B, wl.K, wl.V, code)),
                      t.device)
    out, nacc, am = sd.verify_greedy(t, torch.from_numpy(wl.draft_tokens).cuda(),
                                     k_per_req=None if kp is None else torch.from_numpy(kp).cuda(),
                                     argmax=True, workspace=ws)
    assert_workspace_clean(ws)
    return out.cpu().numpy(), nacc.cpu().numpy(), am.cpu().numpy()


def test_greedy_timed_matches_and_records():
    """specdec_verify_greedy_timed gives the bits of specdec_verify_greedy
    and has the dispatches take the caller's three events."""
    import speculative_decoding_verification_10_amd as sd
    wl = workloads.make("greedy", set_index=1, B=16)
    t = dev_logits(wl.target)
    toks = torch.from_numpy(wl.draft_tokens).cuda()
    ref = sd.verify_greedy(t, toks, argmax=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    got = sd.verify_greedy(t, toks, argmax=True, events=ev)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    assert 0.0 < ev[0].elapsed_time(ev[1]) < ev[0].elapsed_time(ev[2]) < 100.0


def test_greedy_full_size():
    """Fifty distinct seeded sets of the greedy batch (B = 256, K = 3,
    V = 151,936, bf16): argmax, counts and tokens bit-exact."""
    n = 0
    for s, wl, ref in seeded_sets("greedy", 50, ahead=6,
                                  ref_fn=lambda w: oracle.verify_greedy(w.target, w.draft_tokens)):
        if s % 10 == 0:
            say("greedy set", s)
        out, nacc, am = _greedy(wl)
        assert np.array_equal(am, ref["argmax"]), s
        assert np.array_equal(nacc, ref["num_accepted"]), s
        assert np.array_equal(out, ref["out_tokens"]), s
        n += wl.B
    say("counts greedy sets 50 requests", n, "differ 0")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V", [1, 6, 999, 2048, 30001])
def test_greedy_ragged_and_ties(dtype, V):
    rng = np.random.default_rng(V)
    B, K = 40, 5
    # Coarse values make many ties at the max.
    lt = np.round(rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    kp = rng.integers(0, K + 1, size=B).astype(np.int32)
    arr = workloads.bf16_bits(lt) if dtype == "bf16" else lt
    am_true = np.argmax(workloads.stored_as_f32(arr), axis=-1)
    toks = np.where(rng.random((B, K)) < 0.8, am_true[:, :K], rng.integers(0, V, size=(B, K))).astype(np.int32)
    wl = workloads.Workload("g", B, K, V, dtype, 1.0, True, arr, None, toks, np.zeros((B, K + 1), np.float32))
    out, nacc, am = _greedy(wl, kp)
    ref = oracle.verify_greedy(arr, toks, kp)
    assert np.array_equal(am, ref["argmax"])
    assert np.array_equal(nacc, ref["num_accepted"])
    assert np.array_equal(out, ref["out_tokens"])
