"""Helpers shared by the GPU tests: moving seeded workloads to the device and
comparing the HIP path with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from speculative_decoding_verification_10_amd import workloads


def dev_logits(a: np.ndarray, device="cuda") -> torch.Tensor:
    """float32 array or bf16 bit patterns (uint16) -> device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(wl: workloads.Workload, device="cuda") -> dict:
    d = {
        "target": dev_logits(wl.target, device),
        "draft": None if wl.draft is None else dev_logits(wl.draft, device),
        "draft_tokens": torch.from_numpy(wl.draft_tokens).to(device),
        "uniforms": torch.from_numpy(wl.uniforms).to(device),
        "k_per_req": None if wl.k_per_req is None else torch.from_numpy(wl.k_per_req).to(device),
    }
    return d


def compare_verify(name, gpu, ref, rel_tol=1e-5):
    """Tokens and accepted counts bit-exact except on requests the oracle
    flags (a uniform within 1e-6 of a threshold); accept probabilities
    within rel_tol.  Returns (flagged requests, requests that differ; every
    one of the latter is flagged)."""
    out, nacc, ap = gpu
    out = out.cpu().numpy()
    nacc = nacc.cpu().numpy()
    flagged = ref["flagged"]
    ok = ~flagged
    bad_n = np.nonzero(ok & (nacc != ref["num_accepted"]))[0]
    bad_t = np.nonzero(ok & np.any(out != ref["out_tokens"], axis=1))[0]
    assert bad_n.size == 0 and bad_t.size == 0, (
        "%s: %d/%d requests differ outside the flag band, e.g. b=%s gpu=%s oracle=%s margin=%s"
        % (name, max(bad_n.size, bad_t.size), len(nacc),
           (bad_t[:3] if bad_t.size else bad_n[:3]),
           out[(bad_t if bad_t.size else bad_n)[:1]], ref["out_tokens"][(bad_t if bad_t.size else bad_n)[:1]],
           ref["min_margin"][(bad_t if bad_t.size else bad_n)[:1]]))
    if ap is not None:
        ap = ap.cpu().numpy().astype(np.float64)
        rp = ref["accept_prob"]
        used = rp >= 0
        assert np.all(ap[~used] == -1.0), name
        err = np.abs(ap[used] - rp[used]) / np.maximum(np.abs(rp[used]), 1e-30)
        assert err.size == 0 or err.max() < rel_tol, (name, float(err.max()))
    differ = (nacc != ref["num_accepted"]) | np.any(out != ref["out_tokens"], axis=1)
    return int(flagged.sum()), int(differ.sum())


def assert_workspace_clean(ws) -> None:
    """No bounded wait inside the kernels gave up: the workspace's error word,
    read through the C ABI (specdec_workspace_errors), is zero."""
    import speculative_decoding_verification_10_amd as sd
    err = sd.workspace_errors(ws, clear=False)
    assert err == 0, "a wait inside the kernel timed out (error bits %#x)" % err


def run_verify(wl: workloads.Workload, accept_prob=True, device="cuda"):
    import speculative_decoding_verification_10_amd as sd
    d = to_device(wl, device)
    code = 1 if wl.dtype == "bf16" else 0
    ws = sd.Workspace(sd._lib.verify_workspace_bytes(wl.B, wl.K, wl.V, code, wl.draft is None),
                      device)
    res = sd.verify(d["target"], d["draft"], d["draft_tokens"], d["uniforms"], wl.temperature,
                    k_per_req=d["k_per_req"], accept_prob=accept_prob, workspace=ws)
    torch.cuda.synchronize()
    assert_workspace_clean(ws)
    return res


def oracle_verify(wl: workloads.Workload):
    return oracle.verify(wl.target, wl.draft, wl.draft_tokens, wl.uniforms, wl.temperature,
                         wl.k_per_req)


def seeded_sets(name: str, n: int, workers: int = 8, ahead: int = 8, ref_fn=None):
    """Yield (set_index, workload, oracle result) for set_index 0..n-1 of a
    named workload, in order.  Generation and the oracle run in a pool of
    threads (the bulk numpy work releases the GIL), at most `ahead` sets
    ahead of the consumer so host memory stays bounded."""
    from concurrent.futures import ThreadPoolExecutor

    if ref_fn is None:
        ref_fn = oracle_verify

    def build(s):
        wl = workloads.make(name, set_index=s)
        return wl, ref_fn(wl)

    with ThreadPoolExecutor(max_workers=workers) as pool:
        pending = [pool.submit(build, s) for s in range(min(n, ahead))]
        for s in range(n):
            wl, ref = pending[0].result()
            pending.pop(0)
            if s + ahead < n:
                pending.append(pool.submit(build, s + ahead))
            yield s, wl, ref
