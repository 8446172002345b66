"""Checks that pin the CPU oracle to facts outside itself.

Each check takes the oracle module as an argument, so the same battery runs
against the real oracle (every check must pass) and against copies of it with a
planted mistake (at least one check must fail). None of them retypes the
oracle's formulas: they use closed forms, invariants, finite differences, a
scalar brute force written with math.fsum, and torch's CPU float64 softmax and
autograd as an independent library routine.
"""
from __future__ import annotations

import math

import numpy as np

RTOL_EXACT = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


def _max_rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / den


# --- C1: identical keys -------------------------------------------------------
def check_identical_keys(orc):
    rng = _rng(11)
    for causal in (False, True):
        n, d, scale = 9, 4, 0.37
        q = _rand(rng, 1, 1, n, d)
        krow = _rand(rng, d)
        k = np.broadcast_to(krow, (1, 1, n, d)).copy()
        v = _rand(rng, 1, 1, n, d)
        o, lse = orc.attention_forward(q, k, v, causal, scale)
        sc = float(np.float32(scale))
        for i in range(n):
            vis = (i + 1) if causal else n
            assert np.allclose(o[0, 0, i], v[0, 0, :vis].mean(axis=0), rtol=0, atol=1e-12)
            want = sc * float(q[0, 0, i] @ krow) + math.log(vis)
            assert abs(lse[0, 0, i] - want) <= 1e-12 * max(1.0, abs(want))


# --- C2: N = 1 ----------------------------------------------------------------
def check_single_token(orc):
    rng = _rng(12)
    for causal in (False, True):
        q, k, v, do = (_rand(rng, 2, 3, 1, 5) for _ in range(4))
        o, lse = orc.attention_forward(q, k, v, causal, 0.5)
        assert np.array_equal(o, v)
        assert np.allclose(lse, 0.5 * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-14)
        dq, dk, dv = orc.attention_backward(q, k, v, do, causal, 0.5)
        assert np.all(np.abs(dq) <= 1e-15) and np.all(np.abs(dk) <= 1e-15)
        assert np.allclose(dv, do, rtol=0, atol=1e-15)


# --- C3: causal row 0 -------------------------------------------------------
def check_causal_row0(orc):
    rng = _rng(13)
    q, k, v, do = (_rand(rng, 1, 2, 7, 3) for _ in range(4))
    o, lse = orc.attention_forward(q, k, v, True, 0.8)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    sc = float(np.float32(0.8))
    assert np.allclose(lse[:, :, 0], sc * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1),
                       rtol=0, atol=1e-14)
    dq, _, _ = orc.attention_backward(q, k, v, do, True, 0.8)
    assert np.all(np.abs(dq[:, :, 0]) <= 1e-15)


# --- C4: softmax rows are a probability distribution -------------------------
def check_prob_rows(orc):
    rng = _rng(14)
    for causal in (False, True):
        q, k = _rand(rng, 33, 8, sigma=3.0), _rand(rng, 33, 8, sigma=3.0)
        p, lse = orc.head_probs(q, k, causal, 0.3)
        assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 1e-12)
        assert np.all(p >= 0)
        if causal:
            assert np.all(p[np.triu_indices(33, 1)] == 0.0)
            assert np.all(p[np.tril_indices(33)] > 0.0)
        # P_ij = exp(scale * q_i.k_j - LSE_i): the log-sum-exp normalises the row
        sc = float(np.float32(0.3))
        s = sc * (q @ k.T)
        mask = np.tril(np.ones((33, 33), bool)) if causal else np.ones((33, 33), bool)
        assert np.allclose(p[mask], np.exp(s - lse[:, None])[mask], rtol=1e-12, atol=0)


# --- C5: constant V -----------------------------------------------------------
def check_constant_v(orc):
    rng = _rng(15)
    for causal in (False, True):
        q, k = _rand(rng, 1, 2, 10, 4), _rand(rng, 1, 2, 10, 4)
        c = _rand(rng, 4)
        v = np.broadcast_to(c, (1, 2, 10, 4)).copy()
        do = _rand(rng, 1, 2, 10, 4)
        o, _ = orc.attention_forward(q, k, v, causal, 0.6)
        assert np.allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-13)
        dq, dk, _ = orc.attention_backward(q, k, v, do, causal, 0.6)
        assert np.max(np.abs(dq)) <= 1e-13 and np.max(np.abs(dk)) <= 1e-13


# --- C6: permutation equivariance (non-causal) -------------------------------
def check_equivariance(orc):
    rng = _rng(16)
    q, k, v = (_rand(rng, 1, 1, 12, 5) for _ in range(3))
    o, lse = orc.attention_forward(q, k, v, False, 0.45)
    pk = rng.permutation(12)
    o2, lse2 = orc.attention_forward(q, k[:, :, pk], v[:, :, pk], False, 0.45)
    assert np.allclose(o2, o, rtol=0, atol=1e-13) and np.allclose(lse2, lse, rtol=0, atol=1e-13)
    pq = rng.permutation(12)
    o3, lse3 = orc.attention_forward(q[:, :, pq], k, v, False, 0.45)
    assert np.allclose(o3, o[:, :, pq], rtol=0, atol=1e-13)
    assert np.allclose(lse3, lse[:, :, pq], rtol=0, atol=1e-13)


# --- C7: shift invariance of the keys ----------------------------------------
def check_key_shift(orc):
    rng = _rng(17)
    for causal in (False, True):
        q, k, v = (_rand(rng, 1, 1, 11, 6) for _ in range(3))
        u = _rand(rng, 6)
        o, lse = orc.attention_forward(q, k, v, causal, 0.7)
        o2, lse2 = orc.attention_forward(q, k + u, v, causal, 0.7)
        sc = float(np.float32(0.7))
        assert np.allclose(o2, o, rtol=0, atol=1e-12)
        assert np.allclose(lse2, lse + sc * (q[0, 0] @ u)[None, None, :], rtol=0, atol=1e-12)


# --- C8: backward identities --------------------------------------------------
def backward_identities(q, k, v, o, do, dq, dk, dv, scale, causal):
    """Residuals of identities every exact attention backward satisfies, per head.

    Returns a dict of max-normalised residuals:
      sum_j dK_j = 0; sum_j dV_j = sum_i dO_i; <dQ,Q> = <dK,K>.
    (The first holds because each softmax row's dS sums to zero.)
    """
    res = {}
    dk_sum = dk.sum(axis=-2)
    res["sum_dk"] = float(np.max(np.abs(dk_sum))) / max(float(np.max(np.abs(dk))), 1e-300)
    dv_sum, do_sum = dv.sum(axis=-2), do.sum(axis=-2)
    res["sum_dv"] = float(np.max(np.abs(dv_sum - do_sum))) / max(float(np.max(np.abs(do_sum))), 1e-300)
    a = np.einsum("bhnd,bhnd->bh", dq, q)
    b = np.einsum("bhnd,bhnd->bh", dk, k)
    scale_ab = np.maximum(np.einsum("bhnd,bhnd->bh", np.abs(dq), np.abs(q)),
                          np.einsum("bhnd,bhnd->bh", np.abs(dk), np.abs(k)))
    res["qdq_kdk"] = float(np.max(np.abs(a - b) / np.maximum(scale_ab, 1e-300)))
    return res


def check_backward_identities(orc):
    rng = _rng(18)
    for causal in (False, True):
        q, k, v, do = (_rand(rng, 2, 2, 13, 5) for _ in range(4))
        o, _ = orc.attention_forward(q, k, v, causal, 0.55)
        dq, dk, dv = orc.attention_backward(q, k, v, do, causal, 0.55)
        res = backward_identities(q, k, v, o, do, dq, dk, dv, 0.55, causal)
        assert all(r <= 1e-10 for r in res.values()), res
        # and D_i = dO_i . O_i equals sum_j P_ij dP_ij
        for b in range(2):
            for h in range(2):
                p, _ = orc.head_probs(q[b, h], k[b, h], causal, 0.55)
                dp = do[b, h] @ v[b, h].T
                assert np.allclose((p * dp).sum(1), (do[b, h] * o[b, h]).sum(1), rtol=1e-10, atol=1e-12)


# --- C9: finite differences ---------------------------------------------------
def check_finite_differences(orc):
    rng = _rng(19)
    h = 1e-6
    for n in (1, 2, 3, 5, 8):
        for d in (1, 2, 4):
            for causal in (False, True):
                q, k, v, do = (_rand(rng, 1, 2, n, d) for _ in range(4))
                scale = 0.9

                def loss(q_, k_, v_):
                    o_, _ = orc.attention_forward(q_, k_, v_, causal, scale)
                    return float(np.sum(o_ * do))

                grads = orc.attention_backward(q, k, v, do, causal, scale)
                for which, g in enumerate(grads):
                    fd = np.zeros_like(g)
                    args = [q, k, v]
                    for idx in np.ndindex(*g.shape):
                        plus = [a.copy() for a in args]
                        minus = [a.copy() for a in args]
                        plus[which][idx] += h
                        minus[which][idx] -= h
                        fd[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
                    den = max(float(np.max(np.abs(fd))), 1.0)
                    err = float(np.max(np.abs(fd - g))) / den
                    assert err <= 1e-6, (n, d, causal, which, err)


# --- C10: scalar brute force (pure Python) -------------------------------------
def brute_force(q, k, v, do, causal, scale):
    """Attention and its gradient with loops, math.exp and math.fsum only.

    The gradient here goes through the softmax Jacobian written out per entry:
    dL/dS_ij = P_ij * (dO_i . v_j - dO_i . O_i).
    """
    sc = float(np.float32(scale))
    n, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(n)]
    lse = [0.0] * n
    probs = [[0.0] * n for _ in range(n)]
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        s = {j: sc * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in keys}
        m = max(s.values())
        e = {j: math.exp(s[j] - m) for j in keys}
        tot = math.fsum(e.values())
        lse[i] = m + math.log(tot)
        for j in keys:
            probs[i][j] = e[j] / tot
        for c in range(d):
            o[i][c] = math.fsum(probs[i][j] * v[j][c] for j in keys)
    dq = [[0.0] * d for _ in range(n)]
    dk = [[0.0] * d for _ in range(n)]
    dv = [[0.0] * d for _ in range(n)]
    for i in range(n):
        do_o = math.fsum(do[i][c] * o[i][c] for c in range(d))
        for j in range(n):
            pij = probs[i][j]
            if pij == 0.0:
                continue
            do_v = math.fsum(do[i][c] * v[j][c] for c in range(d))
            g = pij * (do_v - do_o)
            for c in range(d):
                dq[i][c] += sc * g * k[j][c]
                dk[j][c] += sc * g * q[i][c]
                dv[j][c] += pij * do[i][c]
    return o, lse, dq, dk, dv


def check_brute_force(orc):
    rng = _rng(20)
    for n in (1, 2, 4, 6):
        for d in (1, 3, 4):
            for causal in (False, True):
                q, k, v, do = (_rand(rng, 1, 1, n, d, sigma=1.5) for _ in range(4))
                o, lse = orc.attention_forward(q, k, v, causal, 0.65)
                dq, dk, dv = orc.attention_backward(q, k, v, do, causal, 0.65)
                bo, blse, bdq, bdk, bdv = brute_force(q[0, 0].tolist(), k[0, 0].tolist(),
                                                      v[0, 0].tolist(), do[0, 0].tolist(),
                                                      causal, 0.65)
                for mine, ref in ((o[0, 0], bo), (lse[0, 0], blse), (dq[0, 0], bdq),
                                  (dk[0, 0], bdk), (dv[0, 0], bdv)):
                    ref = np.asarray(ref)
                    assert np.max(np.abs(mine - ref)) <= 1e-12 * max(1.0, float(np.max(np.abs(ref))))


# --- C11: torch CPU float64 softmax + autograd ---------------------------------
def check_torch_cross(orc):
    import torch
    rng = _rng(21)
    for causal in (False, True):
        for n, d in ((1, 8), (17, 8), (64, 16)):
            q, k, v, do = (_rand(rng, 2, 2, n, d) for _ in range(4))
            scale = float(np.float32(1.0 / math.sqrt(d)))
            tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
            s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
            if causal:
                mask = torch.ones(n, n, dtype=torch.bool).triu(1)
                s = s.masked_fill(mask, float("-inf"))
            to = torch.matmul(torch.softmax(s, dim=-1), tv)
            tlse = torch.logsumexp(s, dim=-1)
            (to * torch.tensor(do)).sum().backward()
            o, lse = orc.attention_forward(q, k, v, causal, scale)
            dq, dk, dv = orc.attention_backward(q, k, v, do, causal, scale)
            for mine, ref in ((o, to.detach().numpy()), (lse, tlse.detach().numpy()),
                              (dq, tq.grad.numpy()), (dk, tk.grad.numpy()), (dv, tv.grad.numpy())):
                assert _max_rel(mine, ref) <= 1e-12, (causal, n, d)


# --- C12: the page's tile recurrence reproduces the two-pass statistics -----
def check_online_recurrence(orc):
    rng = _rng(22)
    for trial in range(50):
        n = int(rng.integers(1, 300))
        x = rng.standard_normal(n) * float(rng.choice([0.1, 1.0, 9.0, 40.0]))
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, int(rng.integers(0, 8))),
                                  replace=False)) if n > 1 else np.array([], int)
        edges = [0, *cuts.tolist(), n]
        tiles = [(edges[t], edges[t + 1]) for t in range(len(edges) - 1)]
        order = rng.permutation(len(tiles))
        m, l = orc.online_softmax_stats(x, [tiles[t] for t in order])
        m_ref = float(x.max())
        l_ref = math.fsum(math.exp(float(t) - m_ref) for t in x)
        assert m == m_ref
        assert abs(l - l_ref) <= 1e-12 * l_ref


# --- bf16 decode --------------------------------------------------------------
def check_bf16_decode(orc):
    import torch
    rng = _rng(23)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    mine = orc.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


# --- binary16 decode ---------------------------------------------------------
def check_f16_decode(orc):
    import torch
    rng = _rng(25)
    bits = np.concatenate([rng.integers(0, 1 << 16, size=4096, dtype=np.uint16),
                           np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0x7C00, 0xFC00,
                                     0x3C00, 0xBC00], dtype=np.uint16)])
    mine = orc.f16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()
    # the smallest subnormal and the largest finite value, from their definitions
    assert mine[-8] == 2.0 ** -24 and mine[-5] == 65504.0 and mine[-4] == np.inf


# --- rows_forward agrees with the full forward ---------------------------------
def check_rows_forward(orc):
    rng = _rng(24)
    for causal in (False, True):
        q, k, v = (_rand(rng, 1, 1, 40, 6) for _ in range(3))
        o, lse = orc.attention_forward(q, k, v, causal, 0.4)
        rows = np.array([0, 1, 7, 39])
        ro, rl = orc.rows_forward(q[0, 0, rows], k[0, 0], v[0, 0], rows, causal, 0.4)
        assert np.allclose(ro, o[0, 0, rows], rtol=0, atol=1e-13)
        assert np.allclose(rl, lse[0, 0, rows], rtol=0, atol=1e-13)


# --- C16: grouped K/V heads against the scalar brute force ---------------------
def check_grouped_heads_brute_force(orc):
    """H query heads over Hkv K/V heads: query head h uses K/V head h Hkv / H
    (consecutive groups), and a K/V head's gradients are the sums over the
    query heads of its group of the single-head brute-force gradients."""
    rng = _rng(26)
    H, d, scale = 6, 3, 0.8
    for Hkv in (1, 2, 3, 6):
        for n in (1, 4, 5):
            for causal in (False, True):
                q, do = (_rand(rng, 1, H, n, d, sigma=1.3) for _ in range(2))
                k, v = (_rand(rng, 1, Hkv, n, d, sigma=1.3) for _ in range(2))
                o, lse = orc.attention_forward(q, k, v, causal, scale)
                dq, dk, dv = orc.attention_backward(q, k, v, do, causal, scale)
                assert dk.shape == k.shape and dv.shape == v.shape
                ref_dk = np.zeros_like(k)
                ref_dv = np.zeros_like(v)
                for h in range(H):
                    g = h * Hkv // H
                    bo, blse, bdq, bdk, bdv = brute_force(q[0, h].tolist(), k[0, g].tolist(),
                                                          v[0, g].tolist(), do[0, h].tolist(),
                                                          causal, scale)
                    for mine, ref in ((o[0, h], bo), (lse[0, h], blse), (dq[0, h], bdq)):
                        ref = np.asarray(ref)
                        assert np.max(np.abs(mine - ref)) <= 1e-12 * max(1.0, float(np.max(np.abs(ref))))
                    ref_dk[0, g] += np.asarray(bdk)
                    ref_dv[0, g] += np.asarray(bdv)
                for mine, ref in ((dk, ref_dk), (dv, ref_dv)):
                    assert np.max(np.abs(mine - ref)) <= 1e-12 * max(1.0, float(np.max(np.abs(ref))))


# --- C17: grouped K/V heads against torch autograd through repeated K/V -------
def check_grouped_heads_torch(orc):
    """Multi-query / grouped-query attention is multi-head attention on K and V
    with each K/V head repeated for the consecutive query heads of its group;
    autograd through torch.repeat_interleave sums the repeated gradients."""
    import torch
    rng = _rng(27)
    B, H, n, d = 2, 8, 9, 4
    for Hkv in (1, 2, 4):
        for causal in (False, True):
            q, do = (_rand(rng, B, H, n, d) for _ in range(2))
            k, v = (_rand(rng, B, Hkv, n, d) for _ in range(2))
            tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
            kr = tk.repeat_interleave(H // Hkv, dim=1)
            vr = tv.repeat_interleave(H // Hkv, dim=1)
            s = torch.matmul(tq, kr.transpose(-1, -2)) * 0.5
            if causal:
                s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
            to = torch.matmul(torch.softmax(s, dim=-1), vr)
            (to * torch.tensor(do)).sum().backward()
            o, lse = orc.attention_forward(q, k, v, causal, 0.5)
            dq, dk, dv = orc.attention_backward(q, k, v, do, causal, 0.5)
            for mine, ref in ((o, to.detach().numpy()),
                              (lse, torch.logsumexp(s, dim=-1).detach().numpy()),
                              (dq, tq.grad.numpy()), (dk, tk.grad.numpy()), (dv, tv.grad.numpy())):
                assert mine.shape == ref.shape
                assert _max_rel(mine, ref) <= 1e-12, (Hkv, causal)


# --- C18: per-key attention mass: closed forms and invariants ----------------
def check_key_mass_closed_forms(orc):
    """Every query row of P sums to 1, so the masses of a batch sum to H N.
    With all keys equal, P is uniform over the visible keys: each key gets
    mass H (non-causal), or H sum_{i >= j} 1 / (i + 1) (causal). The last key
    is seen only by the last query when causal."""
    rng = _rng(28)
    for causal in (False, True):
        for n in (1, 2, 7, 33):
            B, H, Hkv, d = 2, 4, 2, 5
            q = _rand(rng, B, H, n, d)
            k = _rand(rng, B, Hkv, n, d)
            mass = orc.key_mass(q, k, causal, 0.7)
            assert mass.shape == (B, n)
            assert np.allclose(mass.sum(axis=1), H * n, rtol=1e-12, atol=0)
            assert (mass >= 0).all()
            if causal:
                # only query n-1 sees key n-1
                _, lse = orc.attention_forward(q, k, np.eye(n)[None, None].repeat(B, 0).repeat(Hkv, 1),
                                               causal, 0.7)
                sc = float(np.float32(0.7))
                last = np.zeros(B)
                for b in range(B):
                    for h in range(H):
                        g = h * Hkv // H
                        last[b] += math.exp(sc * float(q[b, h, n - 1] @ k[b, g, n - 1]) - lse[b, h, n - 1])
                assert np.allclose(mass[:, n - 1], last, rtol=1e-12, atol=0)
            kc = np.repeat(_rand(rng, B, Hkv, 1, d), n, axis=2)  # identical keys
            mass = orc.key_mass(q, kc, causal, 0.7)
            if causal:
                ref = np.array([H * math.fsum(1.0 / (i + 1) for i in range(j, n)) for j in range(n)])
            else:
                ref = np.full(n, float(H))
            assert np.allclose(mass, ref[None, :], rtol=1e-12, atol=0)


# --- C19: per-key attention mass against torch softmax and a scalar brute force -
def check_key_mass_cross(orc):
    import torch
    rng = _rng(29)
    for causal in (False, True):
        B, H, Hkv, n, d = 2, 6, 3, 11, 4
        q = _rand(rng, B, H, n, d, sigma=1.5)
        k = _rand(rng, B, Hkv, n, d, sigma=1.5)
        tq = torch.tensor(q)
        tk = torch.tensor(k).repeat_interleave(H // Hkv, dim=1)
        s = torch.matmul(tq, tk.transpose(-1, -2)) * float(np.float32(0.45))
        if causal:
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
        ref = torch.softmax(s, dim=-1).sum(dim=(1, 2)).numpy()
        assert _max_rel(orc.key_mass(q, k, causal, 0.45), ref) <= 1e-12
    # scalar brute force (one batch, one head per K/V head)
    for causal in (False, True):
        q = _rand(rng, 1, 2, 5, 3)
        k = _rand(rng, 1, 2, 5, 3)
        mass = orc.key_mass(q, k, causal, 0.9)
        ref = [0.0] * 5
        sc = float(np.float32(0.9))
        for h in range(2):
            for i in range(5):
                keys = range(i + 1) if causal else range(5)
                s = {j: sc * math.fsum(q[0, h, i, c] * k[0, h, j, c] for c in range(3)) for j in keys}
                m = max(s.values())
                tot = math.fsum(math.exp(v - m) for v in s.values())
                for j in keys:
                    ref[j] += math.exp(s[j] - m) / tot
        assert np.max(np.abs(mass[0] - np.asarray(ref))) <= 1e-12 * max(ref)


# --- C20: E4M3 decode and rounding against torch's float8_e4m3fn ------------
def check_e4m3_against_torch(orc):
    """All 256 codes decode as torch's float8_e4m3fn; rounding float32 values
    in [-448, 448] (every grid point, every midpoint between neighbours, and
    random draws at several magnitudes) gives torch's value and byte, zero
    taken as +0."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert ((mine == ref) | (np.isnan(mine) & np.isnan(ref))).all()
    grid = np.unique(mine[np.isfinite(mine)])
    rng = _rng(30)
    ys = np.concatenate([grid, (grid[1:] + grid[:-1]) / 2, rng.uniform(-448, 448, 20000),
                         rng.standard_normal(20000) * 0.02, rng.standard_normal(2000) * 2.0 ** -8])
    ys = ys.astype(np.float32).astype(np.float64)
    r = orc.e4m3_round(ys)
    t = torch.from_numpy(ys.astype(np.float32)).to(torch.float8_e4m3fn)
    tv = t.to(torch.float64).numpy()
    assert np.array_equal(r, np.where(tv == 0, 0.0, tv))
    tb = t.view(torch.uint8).numpy().copy()
    tb[(tb & 0x7F) == 0] = 0
    assert np.array_equal(orc.e4m3_encode(r), tb)
    assert np.array_equal(orc.e4m3_decode(orc.e4m3_encode(r)), r)


# --- C21: block scale exponents: closed forms ---------------------------------
def check_block_exponent(orc):
    """amax = 448 * 2^k needs exactly e = k; anything above it k + 1; half of
    it k - 1; 0 gives 0; tiny blocks stop at -100. On random blocks the
    largest scaled magnitude lands in (224, 448]."""
    for k in (-20, -3, 0, 1, 7, 30):
        a = 448.0 * 2.0 ** k
        assert orc.block_exponent(np.array([a]))[0] == k
        assert orc.block_exponent(np.array([np.nextafter(a, np.inf)]))[0] == k + 1
        assert orc.block_exponent(np.array([a / 2]))[0] == k - 1
        assert orc.block_exponent(np.array([np.nextafter(a / 2, np.inf)]))[0] == k
    assert orc.block_exponent(np.array([0.0]))[0] == 0
    assert orc.block_exponent(np.array([2.0 ** -120]))[0] == -100
    rng = _rng(31)
    x = rng.standard_normal((3, 37, 64)) * np.exp(rng.uniform(-5, 5, (3, 1, 1)))
    _, expo, _ = orc.quantize_e4m3_blocks(x)
    for r in range(3):
        for rb in range(expo.shape[1]):
            for cb in range(expo.shape[2]):
                blk = x[r, 16 * rb:16 * rb + 16, 16 * cb:16 * cb + 16]
                top = np.abs(blk).max() / 2.0 ** expo[r, rb, cb]
                assert 224.0 < top <= 448.0


# --- C22: block quantisation: locality, error bound, fixed points -------------
def check_block_quantisation(orc):
    """Each 16 x 16 block is quantised on its own (changing one element moves
    only its block), the error of a value is at most half an E4M3 step at the
    block's scale, values already on a block's grid are kept exactly, and the
    ragged last row block of a head holds only its own rows."""
    rng = _rng(32)
    R, N, d = 2, 45, 64
    x = rng.standard_normal((R, N, d))
    codes, expo, deq = orc.quantize_e4m3_blocks(x)
    assert codes.shape == (R, N, d) and expo.shape == (R, 3, 4)
    # error bound at the block's scale: |y - y~| <= step / 2 with y = x / 2^e,
    # y~ = x~ / 2^e and step = 2^(max(floor(log2 |y|), -6) - 3)
    scl = 2.0 ** np.repeat(np.repeat(expo, 16, axis=1)[:, :N], 16, axis=2)
    y, yq = x / scl, deq / scl
    _, ex = np.frexp(np.abs(y))
    step = 2.0 ** (np.maximum(ex - 1, -6) - 3)
    assert np.all(np.abs(y - yq) <= step / 2)
    # locality
    x2 = x.copy()
    x2[1, 20, 40] *= 100.0
    c2, e2, _ = orc.quantize_e4m3_blocks(x2)
    changed = np.argwhere(c2 != codes)
    assert len(changed) > 0
    assert set(map(tuple, changed[:, :1])) == {(1,)}
    assert all(16 <= r < 32 and 32 <= c < 48 for _, r, c in changed)
    assert np.argwhere(e2 != expo).tolist() == [[1, 1, 2]]
    # fixed points: E4M3 values times 2^e with a 448 in each block
    grid = orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    z = rng.choice(np.concatenate([grid, -grid]), size=(1, 32, 32)) * 2.0 ** -5
    z[0, ::16, ::16] = 448.0 * 2.0 ** -5
    zc, ze, zd = orc.quantize_e4m3_blocks(z)
    assert np.array_equal(zd, z) and (ze == -5).all()
    assert np.array_equal(orc.e4m3_decode(zc) * 2.0 ** -5, z)
    # idempotent: the dequantised values are their own quantisation
    assert np.array_equal(orc.quantize_e4m3_blocks(deq)[2], deq)
    # the ragged last block: rows 32..44 only
    x3 = x.copy()
    x3[:, 44] = 0.0
    _, e3, d3 = orc.quantize_e4m3_blocks(x3[:, :44])
    assert np.array_equal(d3, orc.quantize_e4m3_blocks(x3)[2][:, :44])


# --- C23: the FP8 forward is exact attention on the dequantised operands -------
def check_fp8_forward(orc):
    """Inputs already on their blocks' grids pass through unchanged, so the
    FP8 forward equals the plain forward there; on general inputs it differs
    from the plain forward by no more than the quantisation of Q and K can
    explain (a first-order bound from |dS| <= |dQ||K| + |Q||dK|)."""
    rng = _rng(33)
    grid = orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    for causal in (False, True):
        q = rng.choice(np.concatenate([grid, -grid]), size=(1, 2, 20, 32)) * 2.0 ** -7
        k = rng.choice(np.concatenate([grid, -grid]), size=(1, 1, 20, 32)) * 2.0 ** -7
        q[..., ::16, ::16] = 448.0 * 2.0 ** -7
        k[..., ::16, ::16] = 448.0 * 2.0 ** -7
        v = rng.standard_normal((1, 1, 20, 32))
        o8, l8 = orc.fp8_attention_forward(q, k, v, causal, 0.3)
        o, lse = orc.attention_forward(q, k, v, causal, 0.3)
        assert np.array_equal(o8, o) and np.array_equal(l8, lse)
        q = rng.standard_normal((2, 4, 33, 32))
        k = rng.standard_normal((2, 2, 33, 32))
        v = rng.standard_normal((2, 2, 33, 32))
        o8, l8 = orc.fp8_attention_forward(q, k, v, causal, 0.3)
        o, lse = orc.attention_forward(q, k, v, causal, 0.3)
        qd = orc.quantize_e4m3_blocks(q.reshape(8, 33, 32))[2].reshape(q.shape)
        kd = orc.quantize_e4m3_blocks(k.reshape(4, 33, 32))[2].reshape(k.shape)
        kr = np.repeat(k, 2, axis=1)
        dkr = np.repeat(np.abs(kd - k), 2, axis=1)
        ds = 0.3 * (np.abs(qd - q) @ np.abs(kr).swapaxes(-1, -2) + np.abs(q) @ dkr.swapaxes(-1, -2))
        bound = ds.max()
        assert 0 < np.abs(l8 - lse).max() <= bound
        assert np.abs(o8 - o).max() <= 2 * bound * np.abs(v).max()
        # quantising is idempotent, so feeding the dequantised Q and K gives
        # the same result: both operands are quantised, and only once
        o8b, l8b = orc.fp8_attention_forward(qd, kd, v, causal, 0.3)
        assert np.array_equal(o8b, o8) and np.array_equal(l8b, l8)
        o8c, _ = orc.fp8_attention_forward(qd, k, v, causal, 0.3)
        o8d, _ = orc.fp8_attention_forward(q, kd, v, causal, 0.3)
        assert np.array_equal(o8c, o8) and np.array_equal(o8d, o8)


# --- C24: 1 x 32 block quantisation: geometry, exponents, error, fixed points --
def check_rows32_quantisation(orc):
    """Each 1 x 32 block (one row, 32 aligned columns) is quantised on its
    own: its exponent is the closed-form one of its own amax (so a block
    whose largest magnitude is 448 * 2^k gets exactly k), changing one
    element moves only its block, the error is at most half an E4M3 step at
    the block's scale, values on a block's grid are kept, and a 16 x 16
    geometry would give other exponents on the same input."""
    rng = _rng(34)
    R, N, d = 2, 7, 128
    x = rng.standard_normal((R, N, d)) * np.exp(rng.uniform(-4, 4, (R, N, 1)))
    codes, expo, deq = orc.quantize_e4m3_rows32(x)
    assert codes.shape == (R, N, d) and expo.shape == (R, N, 4)
    for r in range(R):
        for n in range(N):
            for c in range(4):
                blk = x[r, n, 32 * c:32 * c + 32]
                assert expo[r, n, c] == orc.block_exponent(np.array([np.abs(blk).max()]))[0]
                top = np.abs(blk).max() / 2.0 ** expo[r, n, c]
                assert 224.0 < top <= 448.0
    # closed form: a block whose amax is exactly 448 * 2^k
    z = rng.uniform(-1, 1, (1, 3, 64))
    for n, k in enumerate((-9, 0, 5)):
        z[0, n, :32] *= 448.0 * 2.0 ** k
        z[0, n, 7] = -448.0 * 2.0 ** k
        z[0, n, 32:] = 0.0
    _, ez, dz = orc.quantize_e4m3_rows32(z)
    assert ez[0, :, 0].tolist() == [-9, 0, 5] and (ez[0, :, 1] == 0).all() and (dz[0, :, 32:] == 0).all()
    # error bound
    scl = 2.0 ** np.repeat(expo, 32, axis=2)
    y, yq = x / scl, deq / scl
    _, ex = np.frexp(np.abs(y))
    step = 2.0 ** (np.maximum(ex - 1, -6) - 3)
    assert np.all(np.abs(y - yq) <= step / 2)
    # locality: one element moves only its own 1 x 32 block
    x2 = x.copy()
    x2[1, 4, 70] *= 1000.0
    c2, e2, _ = orc.quantize_e4m3_rows32(x2)
    changed = np.argwhere(c2 != codes)
    assert len(changed) > 0 and all(r == 1 and n == 4 and 64 <= c < 96 for r, n, c in changed)
    assert np.argwhere(e2 != expo).tolist() == [[1, 4, 2]]
    # fixed points and idempotence
    grid = orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    w = rng.choice(np.concatenate([grid, -grid]), size=(1, 4, 64)) * 2.0 ** 3
    w[..., ::32] = 448.0 * 2.0 ** 3
    wc, we, wd = orc.quantize_e4m3_rows32(w)
    assert np.array_equal(wd, w) and (we == 3).all()
    assert np.array_equal(orc.quantize_e4m3_rows32(deq)[2], deq)
    # the geometry matters: 16 x 16 blocks pool 16 rows' magnitudes
    x3 = np.ones((1, 16, 32))
    x3[0, 0, 0] = 448.0 * 2.0 ** 6
    assert orc.quantize_e4m3_rows32(x3)[1][0, 1:, 0].tolist() == [-8] * 15
    assert orc.quantize_e4m3_blocks(x3)[1][0, 0, 0] == 6


# --- C25: the 1 x 32 FP8 forward is exact attention on its dequantised operands
def check_mx_fp8_forward(orc):
    """Inputs on their 1 x 32 blocks' grids pass through unchanged (the
    forward equals the plain one there); on general inputs the result is the
    plain forward of the dequantised Q and K, and differs from the plain
    forward by no more than the quantisation explains; quantising is
    idempotent, so both operands are quantised exactly once."""
    rng = _rng(35)
    grid = orc.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    for causal in (False, True):
        q = rng.choice(np.concatenate([grid, -grid]), size=(1, 2, 20, 64)) * 2.0 ** -7
        k = rng.choice(np.concatenate([grid, -grid]), size=(1, 1, 20, 64)) * 2.0 ** -7
        q[..., ::32] = 448.0 * 2.0 ** -7
        k[..., ::32] = 448.0 * 2.0 ** -7
        v = rng.standard_normal((1, 1, 20, 64))
        o8, l8 = orc.mx_fp8_attention_forward(q, k, v, causal, 0.3)
        o, lse = orc.attention_forward(q, k, v, causal, 0.3)
        assert np.array_equal(o8, o) and np.array_equal(l8, lse)
        q = rng.standard_normal((2, 4, 33, 64))
        k = rng.standard_normal((2, 2, 33, 64))
        v = rng.standard_normal((2, 2, 33, 64))
        o8, l8 = orc.mx_fp8_attention_forward(q, k, v, causal, 0.3)
        qd = orc.quantize_e4m3_rows32(q.reshape(8, 33, 64))[2].reshape(q.shape)
        kd = orc.quantize_e4m3_rows32(k.reshape(4, 33, 64))[2].reshape(k.shape)
        o_d, l_d = orc.attention_forward(qd, kd, v, causal, 0.3)
        assert np.array_equal(o8, o_d) and np.array_equal(l8, l_d)
        o, lse = orc.attention_forward(q, k, v, causal, 0.3)
        kr = np.repeat(k, 2, axis=1)
        dkr = np.repeat(np.abs(kd - k), 2, axis=1)
        ds = 0.3 * (np.abs(qd - q) @ np.abs(kr).swapaxes(-1, -2) + np.abs(q) @ dkr.swapaxes(-1, -2))
        bound = ds.max()
        assert 0 < np.abs(l8 - lse).max() <= bound
        assert np.abs(o8 - o).max() <= 2 * bound * np.abs(v).max()
        o8b, l8b = orc.mx_fp8_attention_forward(qd, kd, v, causal, 0.3)
        assert np.array_equal(o8b, o8) and np.array_equal(l8b, l8)
        # and it is not the 16 x 16 path: with row magnitudes that differ,
        # 16 x 16 blocks share one scale across rows, 1 x 32 blocks do not
        qs = q * np.exp(rng.uniform(-3, 3, (2, 4, 33, 1)))
        assert not np.array_equal(orc.mx_fp8_attention_forward(qs, k, v, causal, 0.3)[0],
                                  orc.fp8_attention_forward(qs, k, v, causal, 0.3)[0])


ALL_CHECKS = [
    check_identical_keys,
    check_single_token,
    check_causal_row0,
    check_prob_rows,
    check_constant_v,
    check_equivariance,
    check_key_shift,
    check_backward_identities,
    check_finite_differences,
    check_brute_force,
    check_torch_cross,
    check_online_recurrence,
    check_bf16_decode,
    check_f16_decode,
    check_rows_forward,
    check_grouped_heads_brute_force,
    check_grouped_heads_torch,
    check_key_mass_closed_forms,
    check_key_mass_cross,
    check_e4m3_against_torch,
    check_block_exponent,
    check_block_quantisation,
    check_fp8_forward,
    check_rows32_quantisation,
    check_mx_fp8_forward,
]
