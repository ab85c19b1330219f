"""GPU parity over seeded random shapes: the stochastic, processed and greedy
verify steps (through the C ABI) against the fp64 oracle, with the batch,
draft length, vocabulary (aligned, odd, tiny, a tile and a ragged tail),
dtype, temperature, logit spread, ties, -inf runs, one-hot drafts, per-request
draft lengths and top-k / top-p drawn together, so that combinations the
targeted tests do not name are covered too."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_verification_10_amd import workloads
from tests.gpu_util import assert_workspace_clean, compare_verify, dev_logits

pytestmark = pytest.mark.gpu

VOCABS = [1, 2, 3, 5, 17, 255, 256, 1000, 2049, 4096, 8191, 8192, 8193, 20000, 65537]
ELEMENTS = 3_000_000          # bound on B * (2K + 1) * V, so the oracle takes seconds

_TALLY = []


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_decoding_verification_10_amd as sd
    sd.load(build_if_missing=False)


def _case(seed):
    """One random configuration: logits (float32 values), drafts, the rest."""
    rng = np.random.default_rng(1000 + seed)
    V = int(rng.choice(VOCABS))
    K = int(rng.integers(0, 11))
    B = int(max(1, min(int(rng.integers(1, 41)), ELEMENTS // ((2 * K + 1) * V))))
    dtype = "bf16" if rng.random() < 0.5 else "fp32"
    T = float(rng.choice([0.3, 0.6, 1.0, 1.7]))
    spread = float(rng.choice([0.1, 1.0, 2.5, 5.0]))
    lt = (rng.standard_normal((B, K + 1, V)) * spread).astype(np.float32)
    if rng.random() < 0.25:                                  # coarse values: many ties
        lt = np.round(lt).astype(np.float32)
    if rng.random() < 0.2 and V > 4:                         # a run of -inf in every row
        a = int(rng.integers(0, V - 2))
        lt[:, :, a:a + int(rng.integers(1, V - a))] = -np.inf
        lt[:, :, V - 1] = np.maximum(lt[:, :, V - 1], 0.0)   # (every row keeps a finite logit)
    one_hot = rng.random() < 0.25
    noise = float(rng.choice([0.0, 0.05, 0.5, 2.0]))
    ld = None                                                # one-hot drafts (and K = 0)
    if not one_hot and K > 0:
        ld = (lt[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32) * noise).astype(np.float32)
        ld[np.isneginf(lt[:, :K])] = -np.inf
    kp = rng.integers(0, K + 1, size=B).astype(np.int32) if (rng.random() < 0.4 and K > 0) else None
    unif = rng.random((B, K + 1), dtype=np.float32)
    return rng, B, K, V, dtype, T, lt, ld, kp, unif


def _stored(a, dtype):
    return None if a is None else (workloads.bf16_bits(a) if dtype == "bf16" else a)


def _draw_tokens(rng, dv, T, B, K, V, kp):
    """Drafts drawn from the draft rows (the q that drew them), else random ids."""
    if dv is None or K == 0:
        return rng.integers(0, max(V, 1), size=(B, K)).astype(np.int32)
    toks = np.zeros((B, K), np.int32)
    for b in range(B):
        kb = K if kp is None else int(kp[b])
        if kb:
            toks[b, :kb] = workloads.gumbel_draw(dv[b, :kb], T, rng)
    return toks


def _run(name, t, d, toks, unif, T, kp, B, K, V, dtype, top_k=None, top_p=None):
    import speculative_decoding_verification_10_amd as sd
    code = 1 if dtype == "bf16" else 0
    processed = top_k is not None
    nbytes = (sd._lib.load().specdec_verify_processed_workspace_bytes(B, K, V, code, int(d is None)) if processed
              else sd._lib.verify_workspace_bytes(B, K, V, code, d is None))
    ws = sd.Workspace(int(nbytes), t.device)
    gpu = sd.verify(t, d, torch.from_numpy(toks).cuda(), torch.from_numpy(unif).cuda(), T,
                    k_per_req=None if kp is None else torch.from_numpy(kp).cuda(), accept_prob=True,
                    workspace=ws, top_k=top_k, top_p=top_p)
    torch.cuda.synchronize()
    assert_workspace_clean(ws)
    return gpu


@pytest.mark.parametrize("seed", range(160))
def test_sweep_verify(seed):
    """The stochastic step, and on every third case the processed step."""
    rng, B, K, V, dtype, T, lt, ld, kp, unif = _case(seed)
    st, sd_ = _stored(lt, dtype), _stored(ld, dtype)
    toks = _draw_tokens(rng, None if sd_ is None else workloads.stored_as_f32(sd_), T, B, K, V, kp)
    say("sweep", seed, dict(B=B, K=K, V=V, dtype=dtype, T=T, one_hot=ld is None, kpr=kp is not None))
    t = dev_logits(st)
    d = None if sd_ is None else dev_logits(sd_)
    gpu = _run("sweep", t, d, toks, unif, T, kp, B, K, V, dtype)
    ref = oracle.verify(st, sd_, toks, unif, T, kp)
    nf, nd = compare_verify("sweep-%d" % seed, gpu, ref)
    _TALLY.append(("verify", seed, nf, nd, B))
    if seed % 3 == 0:
        top_k = int(rng.choice([0, 1, 5, 50, 64, 65, 500]))
        top_p = float(rng.choice([1.0, 0.95, 0.5]))
        if top_k == 0 and top_p == 1.0:
            top_p = 0.8
        if sd_ is not None and K > 0:
            # Drafts redrawn from the processed draft rows.
            dfl, _ = oracle.sampling_floor(sd_, T, top_k, top_p)
            dv = workloads.stored_as_f32(sd_)
            toks = _draw_tokens(rng, np.where(dv >= dfl[..., None], dv, np.float32(-np.inf)), T, B, K, V, kp)
        say("sweep processed", seed, top_k, top_p)
        gpu = _run("sweep-p", t, d, toks, unif, T, kp, B, K, V, dtype, top_k, top_p)
        ref = oracle.verify_processed(st, sd_, toks, unif, T, top_k, top_p, kp)
        nf, nd = compare_verify("sweep-p-%d" % seed, gpu, ref)
        _TALLY.append(("processed", seed, nf, nd, B))


@pytest.mark.parametrize("seed", range(64))
def test_sweep_greedy(seed):
    """The greedy step: argmax, accepted counts and tokens bit-exact."""
    import speculative_decoding_verification_10_amd as sd
    rng, B, K, V, dtype, T, lt, ld, kp, unif = _case(500 + seed)
    st = _stored(lt, dtype)
    am_true = np.argmax(workloads.stored_as_f32(st), axis=-1)
    toks = np.where(rng.random((B, K)) < 0.7, am_true[:, :K], rng.integers(0, V, size=(B, K))).astype(np.int32)
    say("sweep greedy", seed, dict(B=B, K=K, V=V, dtype=dtype, kpr=kp is not None))
    t = dev_logits(st)
    code = 1 if dtype == "bf16" else 0
    ws = sd.Workspace(int(sd._lib.load().specdec_verify_greedy_workspace_bytes(B, K, V, code)), t.device)
    out, nacc, am = sd.verify_greedy(t, torch.from_numpy(toks).cuda(),
                                     k_per_req=None if kp is None else torch.from_numpy(kp).cuda(),
                                     argmax=True, workspace=ws)
    torch.cuda.synchronize()
    assert_workspace_clean(ws)
    ref = oracle.verify_greedy(st, toks, kp)
    assert np.array_equal(am.cpu().numpy(), ref["argmax"])
    assert np.array_equal(nacc.cpu().numpy(), ref["num_accepted"])
    assert np.array_equal(out.cpu().numpy(), ref["out_tokens"])


def test_sweep_mismatch_share():
    """Over the sweep's stochastic and processed cases: requests that differ
    from the oracle (each one flagged, which compare_verify asserted) are at
    most 1 + 10% of the flagged ones."""
    if not _TALLY:
        pytest.skip("no sweep case ran in this session")
    flagged = sum(t[2] for t in _TALLY)
    differ = sum(t[3] for t in _TALLY)
    total = sum(t[4] for t in _TALLY)
    say("counts sweep cases", len(_TALLY), "requests", total, "flagged", flagged, "differ", differ)
    assert differ <= 1 + 0.1 * flagged, (differ, flagged)
