"""GPU parity of the top-k / top-p processed verify step and of the floors
alone: the HIP path (through the C ABI) against the fp64 oracle.  Floors are
compared exactly except on rows whose top-p cut lies within the flag band;
tokens and counts bit-exactly on unflagged requests; accept probabilities
within 1e-5 relative."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_verification_10_amd import workloads
from tests.gpu_util import assert_workspace_clean, compare_verify, dev_logits

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_decoding_verification_10_amd as sd
    sd.load(build_if_missing=False)


def _floors(arr, T, k, p):
    import speculative_decoding_verification_10_amd as sd
    fl = sd.sampling_floors(dev_logits(arr), T, k, p)
    torch.cuda.synchronize()
    ofl, mg = oracle.sampling_floor(arr, T, k, p)
    ok = mg >= oracle.FLAG_BAND
    got = fl.cpu().numpy()
    same = (got == ofl) | (np.isneginf(got) & np.isneginf(ofl))
    bad = np.nonzero(ok & ~same)
    assert bad[0].size == 0, (T, k, p, bad[0][:3], got[bad][:3], ofl[bad][:3])
    return int((~ok).sum()), int((~same).sum())


def _rows(rng, n, V, kind):
    if kind == "normal":
        x = rng.standard_normal((n, V)) * 3
    elif kind == "peaked":
        x = rng.standard_normal((n, V)) * 3
        for r in range(n):
            x[r, rng.choice(V, min(20, V), replace=False)] += 8
    elif kind == "ties":
        x = np.round(rng.standard_normal((n, V)) * 2)
    elif kind == "flat":
        x = rng.standard_normal((n, V)) * 0.05
    elif kind == "zeros":  # mostly -0 and +0, which are one value to every cut
        x = rng.choice(np.array([-0.0, 0.0, -0.0, 0.0, 1.0, -1.0, 2.0]), size=(n, V))
    else:  # "neginf": a third of each row cut to -inf
        x = rng.standard_normal((n, V)) * 2
        x[:, : V // 3] = -np.inf
    return x.astype(np.float32)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("V", [7, 1001, 32000, 128256])
@pytest.mark.parametrize("kind", ["normal", "peaked", "ties", "flat", "neginf", "zeros"])
def test_floors(dtype, V, kind):
    rng = np.random.default_rng(V * 7 + len(kind))
    n = 12 if V > 40000 else 40
    x = _rows(rng, n, V, kind)
    arr = workloads.bf16_bits(x) if dtype == "bf16" else x
    flagged = differ = total = 0
    for T in (1.0, 0.7):
        for k, p in [(0, 1.0), (1, 1.0), (2, 1.0), (50, 1.0), (V - 1, 1.0), (V, 1.0),
                     (0, 0.9), (0, 0.5), (0, 1e-6), (0, 0.999), (40, 0.9), (5000, 0.95),
                     (3, 0.99), (10000, 1.0)]:
            f, d = _floors(arr, T, k, p)
            flagged += f
            differ += d
            total += n
    # A top-p cut near 1 falls among tail tokens of tiny mass, so many rows
    # lie in the flag band there; unflagged rows matched exactly above, and
    # even flagged rows differ only where the masses' rounding decides.
    say(dtype, V, kind, "flagged rows", flagged, "differing", differ, "of", total)
    assert differ <= 0.05 * total, differ


def test_floors_misaligned_rows():
    """An odd vocabulary (scalar loads, a partial last vector) and a row
    start off 16-byte alignment."""
    rng = np.random.default_rng(5)
    x = _rows(rng, 9, 30001, "peaked")
    for arr in (x, workloads.bf16_bits(x)):
        for k, p in [(10, 1.0), (0, 0.8), (100, 0.7)]:
            assert _floors(arr, 0.9, k, p)[1] == 0
    import speculative_decoding_verification_10_amd as sd
    big = dev_logits(np.ascontiguousarray(x.reshape(-1)))
    view = big[3:3 + 8 * 30001 - 3]                      # offset by 12 bytes, 8 rows minus a bit
    rows = view[: (view.numel() // 30001) * 30001].reshape(-1, 30001)
    fl = sd.sampling_floors(rows, 1.0, 10, 0.8)
    torch.cuda.synchronize()
    ofl, mg = oracle.sampling_floor(rows.cpu().numpy(), 1.0, 10, 0.8)
    ok = mg >= oracle.FLAG_BAND
    assert np.array_equal(fl.cpu().numpy()[ok], ofl[ok])


# (case, flagged, differing, requests) of every processed verify case run in
# this module; the last test holds their sum to the mismatch bar.
_TALLY = []


def _processed_case(name, wl, k, p, sets=1):
    """GPU processed verify against the oracle on one workload, with drafts
    redrawn from the processed draft rows (the q that drew them)."""
    import speculative_decoding_verification_10_amd as sd
    T = wl.temperature
    toks = wl.draft_tokens.copy()
    if wl.draft is not None:
        dfl, _ = oracle.sampling_floor(wl.draft, T, k, p)
        dv = workloads.stored_as_f32(wl.draft)
        masked = np.where(dv >= dfl[..., None], dv, np.float32(-np.inf))
        rng = np.random.default_rng(77)
        for b in range(wl.B):
            kb = wl.k_of(b)
            if kb:
                toks[b, :kb] = workloads.gumbel_draw(masked[b, :kb], T, rng)
    t = dev_logits(wl.target)
    d = None if wl.draft is None else dev_logits(wl.draft)
    kp = None if wl.k_per_req is None else torch.from_numpy(wl.k_per_req).cuda()
    code = 1 if wl.dtype == "bf16" else 0
    ws = sd.Workspace(int(sd._lib.load().specdec_verify_processed_workspace_bytes(
        wl.B, wl.K, wl.V, code, int(wl.draft is None))), t.device)
    gpu = sd.verify(t, d, torch.from_numpy(toks).cuda(), torch.from_numpy(wl.uniforms).cuda(), T,
                    k_per_req=kp, accept_prob=True, workspace=ws, top_k=k, top_p=p)
    torch.cuda.synchronize()
    assert_workspace_clean(ws)
    ref = oracle.verify_processed(wl.target, wl.draft, toks, wl.uniforms, T, k, p, wl.k_per_req)
    nf, nd = compare_verify(name, gpu, ref)
    _TALLY.append(("%s k=%d p=%g" % (name, k, p), nf, nd, wl.B))
    say("counts", _TALLY[-1])
    return nf, nd, wl.B


@pytest.mark.parametrize("k,p", [(50, 1.0), (0, 0.9), (40, 0.95), (0, 1.0), (1, 1.0)])
def test_processed_headline_full_size(k, p):
    say("processed headline", k, p)
    wl = workloads.make("headline", set_index=1)
    _processed_case("headline", wl, k, p)


@pytest.mark.parametrize("name", ["peaked", "ragged"])
def test_processed_other_configs(name):
    say("processed", name)
    wl = workloads.make(name, set_index=2, B=64 if name == "ragged" else None)
    for k, p in [(20, 0.9), (0, 0.8)]:
        _processed_case(name, wl, k, p)


def test_processed_tiny_many_steps():
    say("processed tiny x3000")
    wl = workloads.tiny_steps(3000)
    _processed_case("tiny", wl, 10, 0.9)


def test_processed_one_hot_drafts():
    say("processed one-hot")
    wl = workloads.make("greedy", set_index=3, B=32)
    wl.temperature = 0.9
    for k, p in [(5, 1.0), (0, 0.7), (1, 1.0)]:
        _processed_case("one-hot", wl, k, p)


def test_processed_fallback_paths():
    """Cuts the LDS candidates cannot hold (top-k 10,000; top-p over a flat
    row) take the selection over the whole row."""
    wl = workloads.make("peaked", set_index=4)
    nf, nd, B = _processed_case("peaked-k10000", wl, 10000, 1.0)
    assert nd == 0
    rng = np.random.default_rng(9)
    B, K, V = 6, 3, 32000
    lt = (rng.standard_normal((B, K + 1, V)) * 0.05).astype(np.float32)
    ld = (lt[:, :K] + rng.standard_normal((B, K, V)) * 0.05).astype(np.float32)
    flat = workloads.Workload("flat", B, K, V, "fp32", 1.0, False, lt, ld,
                              rng.integers(0, V, (B, K)).astype(np.int32),
                              rng.random((B, K + 1), dtype=np.float32))
    nf, nd, _ = _processed_case("flat-p0.9", flat, 0, 0.9)
    assert nd == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("kind", ["spikes", "ties", "neginf", "normal"])
def test_processed_small_top_k_edges(dtype, kind):
    """A small top-k (at most 64) takes its cuts from each 16 KB tile's
    largest logits; rows whose cut lies below some tile's candidates (a tile
    holding a few far larger logits), coarse ties, a third of each row -inf,
    and top-k 64 / 65 (the limit and past it) against the oracle."""
    rng = np.random.default_rng(31 + len(kind) + (dtype == "bf16"))
    B, K, V = 6, 2, 40000
    lt = (rng.standard_normal((B, K + 1, V)) * 2.0).astype(np.float32)
    if kind == "spikes":
        # A few logits far above the rest in one tile: that tile's candidates
        # stop near its spikes, above the row's top-k cut.
        lt[:, :, 100:103] += 60.0
    elif kind == "ties":
        lt = np.round(lt).astype(np.float32)
    elif kind == "neginf":
        lt[:, :, : V // 3] = -np.inf
    ld = (lt[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32) * 0.5).astype(np.float32)
    if kind == "neginf":
        ld[:, :, : V // 3] = -np.inf
    T = 0.9
    arr_t = workloads.bf16_bits(lt) if dtype == "bf16" else lt
    arr_d = workloads.bf16_bits(ld) if dtype == "bf16" else ld
    toks = rng.integers(0, V, (B, K)).astype(np.int32)
    unif = rng.random((B, K + 1), dtype=np.float32)
    wl = workloads.Workload("edges", B, K, V, dtype, T, False, arr_t, arr_d, toks, unif)
    for k, p in [(1, 1.0), (5, 0.9), (50, 1.0), (50, 0.8), (64, 0.95), (65, 0.9)]:
        _processed_case("edges-%s-%s" % (kind, dtype), wl, k, p)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_processed_small_top_k_many_rows(dtype):
    """More row slots than one round of the combined merge kernel takes
    (1,080 > 1,024): the merge and the full-row path run as two kernels.
    Every request holds a row with spikes in one tile, so rows are left to
    the full-row path there too."""
    rng = np.random.default_rng(57 + (dtype == "bf16"))
    B, K, V = 120, 4, 20000
    lt = (rng.standard_normal((B, K + 1, V)) * 2.0).astype(np.float32)
    lt[:, 1, 300:303] += 60.0
    ld = (lt[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32) * 0.5).astype(np.float32)
    arr_t = workloads.bf16_bits(lt) if dtype == "bf16" else lt
    arr_d = workloads.bf16_bits(ld) if dtype == "bf16" else ld
    wl = workloads.Workload("many", B, K, V, dtype, 0.9, False, arr_t, arr_d,
                            rng.integers(0, V, (B, K)).astype(np.int32), rng.random((B, K + 1), dtype=np.float32))
    for k, p in [(50, 0.9), (8, 1.0)]:
        _processed_case("many-%s" % dtype, wl, k, p)


@pytest.mark.parametrize("dtype,V", [("fp32", 200000), ("bf16", 340000)])
def test_processed_small_top_k_long_rows(dtype, V):
    """Rows of more 16 KB tiles than the merge takes: their small
    top-k cuts come from the full-row path, after the candidates pass."""
    rng = np.random.default_rng(V)
    B, K = 2, 1
    lt = (rng.standard_normal((B, K + 1, V)) * 2.5).astype(np.float32)
    ld = (lt[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32)).astype(np.float32)
    arr_t = workloads.bf16_bits(lt) if dtype == "bf16" else lt
    arr_d = workloads.bf16_bits(ld) if dtype == "bf16" else ld
    wl = workloads.Workload("long", B, K, V, dtype, 0.8, False, arr_t, arr_d,
                            rng.integers(0, V, (B, K)).astype(np.int32), rng.random((B, K + 1), dtype=np.float32))
    for k, p in [(50, 0.9), (10, 1.0)]:
        _processed_case("long-%s" % dtype, wl, k, p)


def test_processed_timed_records_events():
    import speculative_decoding_verification_10_amd as sd
    wl = workloads.make("peaked", set_index=5)
    t = dev_logits(wl.target)
    d = dev_logits(wl.draft)
    toks = torch.from_numpy(wl.draft_tokens).cuda()
    u = torch.from_numpy(wl.uniforms).cuda()
    ref = sd.verify(t, d, toks, u, 1.0, accept_prob=True, top_k=30, top_p=0.9)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    got = sd.verify(t, d, toks, u, 1.0, accept_prob=True, top_k=30, top_p=0.9, events=ev)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    assert 0.0 < ev[0].elapsed_time(ev[1]) < ev[0].elapsed_time(ev[2]) < 100.0


def test_processed_aggregate_mismatch_share():
    """Over every processed case above: requests that differ from the oracle
    (each one flagged, which compare_verify asserted) are at most 0.01% of
    the requests."""
    if not _TALLY:
        pytest.skip("no processed case ran in this session")
    flagged = sum(t[1] for t in _TALLY)
    differ = sum(t[2] for t in _TALLY)
    total = sum(t[3] for t in _TALLY)
    say("counts processed cases", len(_TALLY), "requests", total, "flagged", flagged, "differ", differ)
    assert differ <= 1e-4 * total, (differ, total)
