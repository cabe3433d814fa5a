"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np

import synth

ATOL_O = 2e-2      # max-abs on O against the oracle
ATOL_GRAD = 3e-2   # max-abs on dQ / dK / dV
REL_FRO = 1e-2     # relative Frobenius error per tensor
ATOL_LSE = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def t16(a):
    """bf16 bit array (uint16) -> bf16 CUDA tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())


def i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def host(t):
    return t.float().cpu().numpy()


def compare(name, got, want, atol, rel=REL_FRO, nondegenerate=True):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    nw = float(np.linalg.norm(want))
    r = float(np.linalg.norm(got - want) / nw) if nw > 0 else float(np.linalg.norm(got))
    say(f"  {name}: max-abs {err:.3e} (tol {atol:.0e})  rel-fro {r:.3e} (tol {rel:.0e})  |ref|max {np.max(np.abs(want)) if want.size else 0:.3e}")
    assert err <= atol, f"{name}: max-abs error {err} > {atol}"
    assert r <= rel, f"{name}: relative Frobenius error {r} > {rel}"
    if nondegenerate and nw > 0:
        assert np.linalg.norm(got) >= 0.5 * nw, f"{name}: output norm collapsed"


def fill_pool(pkv, wl, n_pages, bt_np, grads=True, host_tier=False, pool_pages=None, chunk_tokens=65536,
              host_grads=False):
    """Create a pool holding logical pages [0, n_pages) of the workload, appended in pieces."""
    pool = pkv.Pool(pool_pages or len(bt_np), wl.page, wl.h_kv, wl.d, grads=grads, host_tier=host_tier,
                    host_grads=host_grads)
    bt = i32(bt_np)
    per = max(chunk_tokens // wl.page, 1)
    for p0 in range(0, n_pages, per):
        n = min(per, n_pages - p0)
        k, v = synth.kv_tokens(wl, p0, n)
        pool.append(bt, p0 * wl.page, t16(k), t16(v))
    return pool, bt


def scatter_grads(res, L, h_kv, d):
    dk = np.zeros((L, h_kv, d))
    dv = np.zeros((L, h_kv, d))
    for g in range(h_kv):
        np.add.at(dk[:, g, :], res["keys"][g], res["dk"][g])
        np.add.at(dv[:, g, :], res["keys"][g], res["dv"][g])
    return dk, dv
