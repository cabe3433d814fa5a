"""Pins for the attention oracle against things other than itself.

* an independent implementation: PyTorch's scaled_dot_product_attention and autograd, float64, CPU;
* central finite differences of the analytic backward;
* closed forms (first row, identical keys, constant values);
* invariants (chunked == full sequence, sparse == dense over the compacted sequence, selecting
  every page == dense, gradient sums, convex hull).

The sparse key sets (selected pages plus the own block, and one page list per query page) are
written out here as boolean masks from the reading of the pages, never taken from the oracle's own
key-set functions; planted mistakes in those functions must make these pins fail.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _full_grads(res, L, H_kv, d):
    dk = np.zeros((L, H_kv, d))
    dv = np.zeros((L, H_kv, d))
    for g in range(H_kv):
        np.add.at(dk[:, g, :], res["keys"][g], res["dk"][g])
        np.add.at(dv[:, g, :], res["keys"][g], res["dv"][g])
    return dk, dv


def _hand_mask(C, L, q0, P, pages=None):
    """Keys each chunk row may see, written out from the reading of the pages, independently of the
    oracle's own key-set code: with no page list every earlier token; with one, the P tokens of each
    listed page (logical page p holds tokens [p*P, (p+1)*P)) plus the chunk's own block
    [q0, q0 + C); causality (key j <= q0 + t) is applied on top in _torch_reference."""
    allowed = torch.zeros(C, L, dtype=torch.bool)
    if pages is None:
        allowed[:, :] = True
        return allowed
    for p in pages:
        allowed[:, p * P:(p + 1) * P] = True
    allowed[:, q0:q0 + C] = True
    return allowed


def _hand_mask_per_query_page(C, L, q0, P, lists):
    """One page list per query page: the rows of chunk tokens [i*P, (i+1)*P) see lists[i] plus the
    own block."""
    allowed = torch.zeros(C, L, dtype=torch.bool)
    for i, pages in enumerate(lists):
        allowed[i * P:(i + 1) * P] = _hand_mask(C, L, q0, P, pages)[i * P:(i + 1) * P]
    return allowed


def _torch_reference(q, k, v, do, q0, scale, masks, H_q, H_kv):
    """Independent reference with torch SDPA (math path) + autograd, float64.

    masks[g]: [C][L] boolean, the keys each row of KV head g's query heads may see before the
    causal cut."""
    C, _, d = q.shape
    L = k.shape[0]
    G = H_q // H_kv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    outs = []
    for h in range(H_q):
        g = h // G
        qpos = torch.arange(C) + q0
        allowed = masks[g].clone() & (torch.arange(L)[None, :] <= qpos[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(
            tq[:, h, :][None, None], tk[:, g, :][None, None], tv[:, g, :][None, None],
            attn_mask=allowed[None, None], scale=scale)
        outs.append(o[0, 0])
    out = torch.stack(outs, dim=1)
    loss = (out * torch.tensor(do, dtype=torch.float64)).sum()
    loss.backward()
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("sparse", [False, True])
def test_matches_torch_sdpa_and_autograd(sparse):
    rng = np.random.default_rng(7)
    H_q, H_kv, d, P, C = 4, 2, 8, 4, 16
    n_prior = 10
    q0 = n_prior * P
    L = q0 + C
    q, k, v, do = _rand((C, H_q, d), rng), _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng), _rand((C, H_q, d), rng)
    scale = 0.37
    sel = [[1, 4, 7], [0, 8, 9]] if sparse else None
    o, lse = oracle.chunk_forward(q, k, v, q0, scale, sel=sel, page=P)
    res = oracle.chunk_backward(q, k, v, do, q0, scale, sel=sel, page=P)
    masks = [_hand_mask(C, L, q0, P, None if sel is None else sel[g]) for g in range(H_kv)]
    to, tdq, tdk, tdv = _torch_reference(q, k, v, do, q0, scale, masks, H_q, H_kv)
    dk, dv = _full_grads(res, L, H_kv, d)
    assert np.max(np.abs(o - to)) < 1e-12
    assert np.max(np.abs(res["dq"] - tdq)) < 1e-12
    assert np.max(np.abs(dk - tdk)) < 1e-12
    assert np.max(np.abs(dv - tdv)) < 1e-12
    # LSE against a direct log-sum-exp of the masked scores.
    for h in range(H_q):
        g = h // (H_q // H_kv)
        for t in range(C):
            ks = [j for j in range(L) if masks[g][t, j] and j <= q0 + t]
            s = scale * np.array([q[t, h] @ k[j, g] for j in ks])
            assert abs(lse[h, t] - (s.max() + np.log(np.exp(s - s.max()).sum()))) < 1e-12


def test_finite_differences():
    rng = np.random.default_rng(3)
    H_q, H_kv, d, P, C = 4, 2, 6, 4, 8
    q0 = 8
    L = q0 + C
    q, k, v, do = _rand((C, H_q, d), rng), _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng), _rand((C, H_q, d), rng)
    scale = 0.5

    def loss(q_, k_, v_):
        o, _ = oracle.chunk_forward(q_, k_, v_, q0, scale, page=P)
        return float((o * do).sum())

    res = oracle.chunk_backward(q, k, v, do, q0, scale, page=P)
    dk, dv = _full_grads(res, L, H_kv, d)
    eps = 1e-5
    picks = [(a, tuple(rng.integers(0, s) for s in arr.shape)) for a, arr in
             [("q", q), ("k", k), ("v", v)] for _ in range(12)]
    for name, idx in picks:
        arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
        arrs[name][idx] += eps
        up = loss(arrs["q"], arrs["k"], arrs["v"])
        arrs[name][idx] -= 2 * eps
        dn = loss(arrs["q"], arrs["k"], arrs["v"])
        fd = (up - dn) / (2 * eps)
        an = {"q": res["dq"], "k": dk, "v": dv}[name][idx]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)


def test_closed_forms():
    rng = np.random.default_rng(11)
    H_q, H_kv, d, C = 2, 1, 5, 12
    q, v, do = _rand((C, H_q, d), rng), _rand((C, H_kv, d), rng), _rand((C, H_q, d), rng)
    k = _rand((C, H_kv, d), rng)
    s = 0.3
    # Row 0 of a sequence sees only key 0: O = v0, LSE = s q0.k0.
    o, lse = oracle.chunk_forward(q, k, v, 0, s, page=4)
    for h in range(H_q):
        assert np.allclose(o[0, h], v[0, 0], atol=1e-15)
        assert abs(lse[h, 0] - s * q[0, h] @ k[0, 0]) < 1e-14
    # All keys equal: uniform weights -> prefix mean of V, LSE = s q.k + log(t+1).
    kc = np.repeat(k[:1], C, axis=0)
    o, lse = oracle.chunk_forward(q, kc, v, 0, s, page=4)
    for t in range(C):
        assert np.allclose(o[t, 0], v[: t + 1, 0].mean(axis=0), atol=1e-14)
        assert abs(lse[0, t] - (s * q[t, 0] @ kc[0, 0] + np.log(t + 1))) < 1e-13
    # Constant V: O = v, dQ = dK = 0, sum_j dV_j = sum_t dO_t.
    vc = np.repeat(v[:1], C, axis=0)
    res = oracle.chunk_backward(q, k, vc, do, 0, s, page=4)
    assert np.allclose(res["o"], np.broadcast_to(vc[0, 0], res["o"].shape), atol=1e-14)
    assert np.max(np.abs(res["dq"])) < 1e-13 and np.max(np.abs(res["dk"][0])) < 1e-13
    assert np.allclose(res["dv"][0].sum(axis=0), do.sum(axis=(0, 1)), atol=1e-12)


def test_invariants_and_chunking():
    rng = np.random.default_rng(5)
    H_q, H_kv, d, P = 6, 2, 8, 8
    L, C = 64, 16
    q_full, k, v, do_full = (_rand((L, H_q, d), rng), _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng),
                             _rand((L, H_q, d), rng))
    s = 1 / np.sqrt(d)
    full = oracle.chunk_backward(q_full, k, v, do_full, 0, s, page=P)
    dk_full, dv_full = _full_grads(full, L, H_kv, d)
    dk_acc = np.zeros_like(dk_full)
    dv_acc = np.zeros_like(dv_full)
    for c in range(L // C):
        sl = slice(c * C, (c + 1) * C)
        r = oracle.chunk_backward(q_full[sl], k, v, do_full[sl], c * C, s, page=P)
        o, lse = oracle.chunk_forward(q_full[sl], k, v, c * C, s, page=P)
        assert np.max(np.abs(o - full["o"][sl])) < 1e-13
        assert np.max(np.abs(lse - full["lse"][:, sl])) < 1e-13
        assert np.max(np.abs(r["dq"] - full["dq"][sl])) < 1e-13
        a, b = _full_grads(r, L, H_kv, d)
        dk_acc += a
        dv_acc += b
        # Per call and KV head: sum_j dV_j = sum over the group's rows of dO; sum_j dK_j = 0.
        G = H_q // H_kv
        for g in range(H_kv):
            assert np.allclose(r["dv"][g].sum(axis=0), do_full[sl, g * G:(g + 1) * G].sum(axis=(0, 1)), atol=1e-12)
            assert np.max(np.abs(r["dk"][g].sum(axis=0))) < 1e-12
        # Each output row lies in the convex hull (per dimension) of the values it sees.
        for t in range(C):
            seen = v[: c * C + t + 1]
            for h in range(H_q):
                g = h // G
                assert np.all(o[t, h] <= seen[:, g].max(axis=0) + 1e-12)
                assert np.all(o[t, h] >= seen[:, g].min(axis=0) - 1e-12)
    assert np.max(np.abs(dk_acc - dk_full)) < 1e-12
    assert np.max(np.abs(dv_acc - dv_full)) < 1e-12


def test_sparse_equals_dense_over_compacted_sequence():
    rng = np.random.default_rng(9)
    H_q, H_kv, d, P, C = 4, 1, 8, 4, 8
    n_prior = 9
    q0 = n_prior * P
    L = q0 + C
    q, k, v, do = _rand((C, H_q, d), rng), _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng), _rand((C, H_q, d), rng)
    sel = [[0, 3, 4, 8]]
    s = 0.4
    o, lse = oracle.chunk_forward(q, k, v, q0, s, sel=sel, page=P)
    res = oracle.chunk_backward(q, k, v, do, q0, s, sel=sel, page=P)
    # The compacted key sequence written out by hand: the selected pages' tokens, then the own block.
    toks = np.concatenate([np.arange(p * P, (p + 1) * P) for p in sel[0]] + [np.arange(q0, q0 + C)])
    assert np.array_equal(toks, oracle.visible_keys(q0, C, P, sel[0]))
    kc, vc = k[toks], v[toks]
    q0c = len(sel[0]) * P
    oc, lsec = oracle.chunk_forward(q, kc, vc, q0c, s, page=P)
    rc = oracle.chunk_backward(q, kc, vc, do, q0c, s, page=P)
    assert np.max(np.abs(o - oc)) < 1e-13 and np.max(np.abs(lse - lsec)) < 1e-13
    assert np.max(np.abs(res["dq"] - rc["dq"])) < 1e-13
    assert np.max(np.abs(res["dk"][0] - rc["dk"][0])) < 1e-13
    # Selecting every prior page is exactly dense attention (same key order, bitwise).
    allsel = [list(range(n_prior))]
    o_all, lse_all = oracle.chunk_forward(q, k, v, q0, s, sel=allsel, page=P)
    o_d, lse_d = oracle.chunk_forward(q, k, v, q0, s, page=P)
    assert np.array_equal(o_all, o_d) and np.array_equal(lse_all, lse_d)


def test_paged_permutation_invariance():
    """A paged store (pages scattered by a random block table) read back through the table gives
    the same oracle results as the contiguous sequence."""
    rng = np.random.default_rng(2)
    H_q, H_kv, d, P, C = 4, 2, 8, 8, 16
    L = 64
    k, v = _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng)
    q, do = _rand((C, H_q, d), rng), _rand((C, H_q, d), rng)
    n_pages = L // P
    bt = rng.permutation(n_pages)
    pool = np.zeros((n_pages, H_kv, 2, P, d))
    for lp in range(n_pages):
        pool[bt[lp], :, 0] = k[lp * P:(lp + 1) * P].transpose(1, 0, 2)
        pool[bt[lp], :, 1] = v[lp * P:(lp + 1) * P].transpose(1, 0, 2)
    kg = np.concatenate([pool[bt[lp], :, 0].transpose(1, 0, 2) for lp in range(n_pages)])
    vg = np.concatenate([pool[bt[lp], :, 1].transpose(1, 0, 2) for lp in range(n_pages)])
    q0 = L - C
    a = oracle.chunk_forward(q, k, v, q0, 0.3, page=P)
    b = oracle.chunk_forward(q, kg, vg, q0, 0.3, page=P)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_float32_mode_close_to_float64():
    rng = np.random.default_rng(4)
    H_q, H_kv, d, P, C = 4, 1, 64, 64, 64
    q0 = 256
    L = q0 + C
    q, k, v = _rand((C, H_q, d), rng), _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng)
    s = 0.125
    o64, l64 = oracle.chunk_forward(q, k, v, q0, s, page=P)
    o32, l32 = oracle.chunk_forward(q, k, v, q0, s, page=P, dtype=np.float32)
    assert o32.dtype == np.float32
    assert np.max(np.abs(o64 - o32)) < 1e-5 and np.max(np.abs(l64 - l32)) < 1e-5


def test_bf16_bits_accepted():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((8, 4)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    w = oracle.widen_bf16(bits)
    assert w.dtype == np.float32
    assert np.array_equal(w.view(np.uint32) & 0xFFFF, np.zeros_like(bits, dtype=np.uint32))
    assert np.max(np.abs(w - x)) <= np.max(np.abs(x)) * 2 ** -7


def test_per_query_page_lists_match_torch_sdpa_and_autograd():
    """One page list per query page (pt 2.C): every row sees its own query page's pages plus the
    own block, checked against SDPA with the per-row mask written out."""
    rng = np.random.default_rng(11)
    H_q, H_kv, d, P, C = 4, 2, 8, 4, 16
    n_prior = 10
    q0 = n_prior * P
    L = q0 + C
    q, k, v, do = _rand((C, H_q, d), rng), _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng), _rand((C, H_q, d), rng)
    scale = 0.37
    sel = np.array([[[1, 4, 7], [0, 2, 9], [5, 6, 8], [1, 3, 4]],
                    [[0, 8, 9], [2, 3, 7], [4, 5, 9], [0, 1, 6]]])
    o, lse = oracle.chunk_forward(q, k, v, q0, scale, sel=sel, page=P)
    res = oracle.chunk_backward(q, k, v, do, q0, scale, sel=sel, page=P)
    masks = [_hand_mask_per_query_page(C, L, q0, P, sel[g]) for g in range(H_kv)]
    to, tdq, tdk, tdv = _torch_reference(q, k, v, do, q0, scale, masks, H_q, H_kv)
    dk, dv = _full_grads(res, L, H_kv, d)
    assert np.max(np.abs(o - to)) < 1e-12
    assert np.max(np.abs(res["o"] - to)) < 1e-12
    assert np.max(np.abs(res["dq"] - tdq)) < 1e-12
    assert np.max(np.abs(dk - tdk)) < 1e-12
    assert np.max(np.abs(dv - tdv)) < 1e-12
    # Keys no list selects get no gradient; the reported keys are the union, ascending.
    for g in range(H_kv):
        want = np.nonzero(masks[g].any(dim=0).numpy())[0]
        assert np.array_equal(res["keys"][g], want)
    # A row subset returns the same rows.
    rows = np.array([1, 6, 13])
    o2, lse2 = oracle.chunk_forward(q, k, v, q0, scale, sel=sel, page=P, rows=rows)
    assert np.max(np.abs(o2 - o[rows])) < 1e-13 and np.max(np.abs(lse2 - lse[:, rows])) < 1e-13


def test_per_query_page_identical_lists_equal_one_list():
    rng = np.random.default_rng(12)
    H_q, H_kv, d, P, C = 4, 2, 8, 4, 16
    n_prior = 10
    q0 = n_prior * P
    L = q0 + C
    q, k, v, do = _rand((C, H_q, d), rng), _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng), _rand((C, H_q, d), rng)
    sel2 = [[1, 4, 7], [0, 8, 9]]
    sel3 = np.repeat(np.array(sel2)[:, None, :], C // P, axis=1)
    o2, l2 = oracle.chunk_forward(q, k, v, q0, 0.3, sel=sel2, page=P)
    o3, l3 = oracle.chunk_forward(q, k, v, q0, 0.3, sel=sel3, page=P)
    assert np.max(np.abs(o2 - o3)) < 1e-13 and np.max(np.abs(l2 - l3)) < 1e-13
    r2 = oracle.chunk_backward(q, k, v, do, q0, 0.3, sel=sel2, page=P)
    r3 = oracle.chunk_backward(q, k, v, do, q0, 0.3, sel=sel3, page=P)
    assert np.max(np.abs(r2["dq"] - r3["dq"])) < 1e-13
    for g in range(H_kv):
        assert np.array_equal(r2["keys"][g], r3["keys"][g])
        assert np.max(np.abs(r2["dk"][g] - r3["dk"][g])) < 1e-12
        assert np.max(np.abs(r2["dv"][g] - r3["dv"][g])) < 1e-12


# Planted mistakes in the oracle's key-set code (on the CPU, in this process only): each must make
# the hand-masked SDPA pin above fail, so the pin really constrains which keys the oracle uses.
def _broken_visible_keys_no_page_scale(q0, chunk, page, sel_pages=None):
    if sel_pages is None:
        return np.arange(q0 + chunk, dtype=np.int64)
    sel = np.asarray(sel_pages, dtype=np.int64).reshape(-1)
    toks = (sel[:, None] + np.arange(page, dtype=np.int64)[None, :]).reshape(-1)  # page id not scaled
    return np.concatenate([toks, np.arange(q0, q0 + chunk, dtype=np.int64)])


def _broken_visible_keys_own_block_shift(q0, chunk, page, sel_pages=None):
    if sel_pages is None:
        return np.arange(q0 + chunk, dtype=np.int64)
    sel = np.asarray(sel_pages, dtype=np.int64).reshape(-1)
    toks = (sel[:, None] * page + np.arange(page, dtype=np.int64)[None, :]).reshape(-1)
    return np.concatenate([toks, np.arange(q0 + 1, q0 + chunk, dtype=np.int64)])  # own block off by one


def _broken_visible_keys_no_own_block(q0, chunk, page, sel_pages=None):
    if sel_pages is None:
        return np.arange(q0 + chunk, dtype=np.int64)
    sel = np.asarray(sel_pages, dtype=np.int64).reshape(-1)
    return (sel[:, None] * page + np.arange(page, dtype=np.int64)[None, :]).reshape(-1)


def _broken_visible_keys_page_shift(q0, chunk, page, sel_pages=None):
    if sel_pages is None:
        return np.arange(q0 + chunk, dtype=np.int64)
    sel = np.asarray(sel_pages, dtype=np.int64).reshape(-1) + 1  # every selected page one later
    toks = (sel[:, None] * page + np.arange(page, dtype=np.int64)[None, :]).reshape(-1)
    return np.concatenate([toks, np.arange(q0, q0 + chunk, dtype=np.int64)])


def _sparse_pin_errors(sel):
    """Max-abs differences between the oracle and the hand-masked SDPA reference on one sparse case
    (O, dQ, dK, dV), with the oracle as it currently stands in this process."""
    rng = np.random.default_rng(21)
    H_q, H_kv, d, P, C = 4, 2, 8, 4, 16
    n_prior = 10
    q0 = n_prior * P
    L = q0 + C
    q, k, v, do = _rand((C, H_q, d), rng), _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng), _rand((C, H_q, d), rng)
    scale = 0.37
    res = oracle.chunk_backward(q, k, v, do, q0, scale, sel=sel, page=P)
    if np.ndim(sel[0]) == 1:
        masks = [_hand_mask(C, L, q0, P, sel[g]) for g in range(H_kv)]
    else:
        masks = [_hand_mask_per_query_page(C, L, q0, P, sel[g]) for g in range(H_kv)]
    to, tdq, tdk, tdv = _torch_reference(q, k, v, do, q0, scale, masks, H_q, H_kv)
    dk, dv = _full_grads(res, L, H_kv, d)
    return max(np.max(np.abs(res["o"] - to)), np.max(np.abs(res["dq"] - tdq)), np.max(np.abs(dk - tdk)),
               np.max(np.abs(dv - tdv)))


_SEL_SHARED = [[1, 4, 7], [0, 8, 9]]
_SEL_PER_QPAGE = np.array([[[1, 4, 7], [0, 2, 9], [5, 6, 8], [1, 3, 4]],
                           [[0, 8, 9], [2, 3, 7], [4, 5, 9], [0, 1, 6]]])


@pytest.mark.parametrize("broken", [_broken_visible_keys_no_page_scale, _broken_visible_keys_own_block_shift,
                                    _broken_visible_keys_no_own_block, _broken_visible_keys_page_shift])
@pytest.mark.parametrize("sel", [_SEL_SHARED, _SEL_PER_QPAGE], ids=["shared", "per_query_page"])
def test_planted_key_set_mistakes_fail_the_pin(monkeypatch, broken, sel):
    assert _sparse_pin_errors(sel) < 1e-12
    monkeypatch.setattr(oracle.attention, "visible_keys", broken)
    err = _sparse_pin_errors(sel)
    assert err > 1e-3, f"planted mistake {broken.__name__} went unnoticed (error {err})"


def _broken_key_sets_list_per_row_block(q0, C, page, sel, g, rows):
    """Per-query-page routing with the query page of a row computed from the wrong page size."""
    lists = np.asarray(sel[g])
    if lists.ndim == 1:
        yield oracle.attention.visible_keys(q0, C, page, lists), np.arange(len(rows))
        return
    qpage = np.minimum(rows // (2 * page), lists.shape[0] - 1)
    for i in range(lists.shape[0]):
        pos = np.nonzero(qpage == i)[0]
        if len(pos):
            yield oracle.attention.visible_keys(q0, C, page, lists[i]), pos


def _broken_key_sets_first_list_only(q0, C, page, sel, g, rows):
    """Every row routed to the first query page's list."""
    lists = np.asarray(sel[g])
    first = lists if lists.ndim == 1 else lists[0]
    yield oracle.attention.visible_keys(q0, C, page, first), np.arange(len(rows))


@pytest.mark.parametrize("broken", [_broken_key_sets_list_per_row_block, _broken_key_sets_first_list_only])
def test_planted_per_query_page_routing_mistakes_fail_the_pin(monkeypatch, broken):
    assert _sparse_pin_errors(_SEL_PER_QPAGE) < 1e-12
    monkeypatch.setattr(oracle.attention, "_key_sets", broken)
    assert _sparse_pin_errors(_SEL_PER_QPAGE) > 1e-3


@pytest.mark.parametrize("sparse", [False, True])
def test_key_gradients_from_row_statistics_match_torch_autograd(sparse):
    """dK/dV of a few keys, from the forward's LSE and D = dO.O, equal the gradients SDPA's autograd
    gives those keys (dense, and a shared page list whose pages plus the own block every row sees)."""
    rng = np.random.default_rng(17)
    H_q, H_kv, d, P, C = 6, 2, 8, 4, 16
    n_prior = 10
    q0 = n_prior * P
    L = q0 + C
    q, k, v, do = _rand((C, H_q, d), rng), _rand((L, H_kv, d), rng), _rand((L, H_kv, d), rng), _rand((C, H_q, d), rng)
    scale = 0.41
    sel = [[1, 4, 7], [0, 8, 9]] if sparse else None
    o, lse = oracle.chunk_forward(q, k, v, q0, scale, sel=sel, page=P)
    dd = np.einsum("thd,thd->ht", do, o)
    masks = [_hand_mask(C, L, q0, P, None if sel is None else sel[g]) for g in range(H_kv)]
    _, _, tdk, tdv = _torch_reference(q, k, v, do, q0, scale, masks, H_q, H_kv)
    # Keys from a prior page, the first own-block key (seen by every row) and the last one (seen by
    # the last row only), written out by hand per head.
    keys = {0: np.array([4 * P, 4 * P + 3, q0, q0 + C - 1]) if sparse else np.array([0, 17, q0, q0 + C - 1]),
            1: np.array([8 * P + 1, 9 * P + 2, q0 + 5]) if sparse else np.array([3, 39, q0 + 5])}
    got = oracle.key_gradients(q, k, v, do, q0, scale, keys, lse, dd)
    for g, kidx in keys.items():
        assert np.max(np.abs(got[g][0] - tdk[kidx, g])) < 1e-12
        assert np.max(np.abs(got[g][1] - tdv[kidx, g])) < 1e-12
        assert np.max(np.abs(got[g][0])) > 1e-3  # not vacuous
