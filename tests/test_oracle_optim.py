"""Pins for the oracle's update rules and full fused step (CPU only).

Anchors: torch.optim.AdamW / torch.optim.SGD in float64 (a library routine),
a float64 textbook loop written here, the first-step closed form, the
update's float32 arithmetic against exact rationals rounded once per
operation (inputs chosen where multiplying by a rounded reciprocal instead of
dividing changes the result), the bf16 + 16-bit ECC identity (a lossless
split must reproduce a plain float32 master bit for bit), and the storage
byte count the pages give.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from oracle.optim import fresh_adamw_state, fresh_sgdm_state

from exact_fp import f32, rn32, rn32_sqrt

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _torch_adamw(x0, grads, hp):
    p = torch.nn.Parameter(torch.tensor(x0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    out = []
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        out.append(p.detach().numpy().copy())
    return out


def _oracle_unquantised_adamw(x0, grads, hp):
    th = x0.astype(np.float32)
    m = np.zeros_like(th); v = np.zeros_like(th)
    out = []
    for t, g in enumerate(grads, start=1):
        S = O.adamw_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], t)
        th, m, v, _ = O.adamw_update(th, g.astype(np.float32), m, v, S)
        out.append(th.copy())
    return out


def _textbook_adamw(x0, grads, hp):
    # plain float64 AdamW, written from the textbook definition
    th = x0.astype(np.float64); m = np.zeros_like(th); v = np.zeros_like(th)
    out = []
    for t, g in enumerate(grads, start=1):
        g = g.astype(np.float64)
        th = th - hp["lr"] * hp["weight_decay"] * th
        m = hp["beta1"] * m + (1 - hp["beta1"]) * g
        v = hp["beta2"] * v + (1 - hp["beta2"]) * g * g
        mh = m / (1 - hp["beta1"] ** t)
        vh = v / (1 - hp["beta2"] ** t)
        th = th - hp["lr"] * mh / (np.sqrt(vh) + hp["eps"])
        out.append(th.copy())
    return out


@pytest.mark.parametrize("hp", [HP, dict(lr=6e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)])
def test_unquantised_adamw_matches_torch_and_textbook(hp):
    rng = np.random.default_rng(20)
    x0 = (rng.standard_normal((7, 5)) * 0.02).astype(np.float32)
    grads = [(rng.standard_t(3, (7, 5)) * 1e-3).astype(np.float32) for _ in range(10)]
    a = _oracle_unquantised_adamw(x0, grads, hp)
    b = _torch_adamw(x0.astype(np.float64), [g.astype(np.float64) for g in grads], hp)
    c = _textbook_adamw(x0, grads, hp)
    # float32 trajectory vs float64 references: normwise 1e-6, and the
    # accumulated update itself within 1e-4 (a dropped bias correction, a
    # wrong sign or a misplaced eps changes it by far more)
    for x, y, z in zip(a, b, c):
        for ref in (y, z):
            assert np.max(np.abs(x - ref)) <= 1e-6 * np.max(np.abs(ref))
            assert np.max(np.abs((x - x0) - (ref - x0))) <= 1e-4 * np.max(np.abs(ref - x0))


def test_unquantised_sgdm_matches_torch():
    rng = np.random.default_rng(21)
    x0 = (rng.standard_normal((7, 5)) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal((7, 5)) * 1e-2).astype(np.float32) for _ in range(10)]
    p = torch.nn.Parameter(torch.tensor(x0, dtype=torch.float64))
    opt = torch.optim.SGD([p], lr=0.1, momentum=0.9, weight_decay=1e-4, foreach=False)
    S = O.sgdm_scalars(0.1, 0.9, 1e-4)
    th = x0.copy(); b = np.zeros_like(th)
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        th, b = O.sgdm_update(th, g, b, S)
        ref = p.detach().numpy()
        assert np.max(np.abs(th - ref)) <= 1e-6 * np.max(np.abs(ref))
        assert np.max(np.abs((th - x0) - (ref - x0))) <= 1e-4 * np.max(np.abs(ref - x0))


def test_first_step_closed_form():
    # from zero states, m = (1-b1) g and v = (1-b2) g^2, so the update is
    # lr * g / (|g| + eps*sqrt(1-b2)/(1-b1)...) ~= lr * sign(g) for |g| >> eps
    rng = np.random.default_rng(22)
    th0 = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    g = (rng.standard_t(3, 1000) * 1e-3).astype(np.float32)
    S = O.adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    th, m, v, _ = O.adamw_update(th0, g, np.zeros(1000, np.float32), np.zeros(1000, np.float32), S)
    big = np.abs(g) > 1e-5
    assert np.allclose((th0 - th)[big], 1e-3 * np.sign(g[big]), rtol=2e-3, atol=0)
    assert np.array_equal(m, np.float32(0.9) * np.float32(0) + np.float32(1.0 - 0.9) * g)


def _run_ecc16_vs_plain(fmt_bits=16, steps=8):
    # bf16 + 16-bit ECC is lossless, so storing the master as (theta', rho)
    # between steps must reproduce a plain float32 master bit for bit.
    rng = np.random.default_rng(23)
    x0 = (rng.standard_normal(4096) * 0.02).astype(np.float32)
    plain = x0.copy(); m1 = np.zeros_like(x0); v1 = np.zeros_like(x0)
    w16, ecc = O.split_weights(x0, "bf16", fmt_bits)
    m2 = np.zeros_like(x0); v2 = np.zeros_like(x0)
    for t in range(1, steps + 1):
        g = (rng.standard_t(3, 4096) * 1e-3).astype(np.float32)
        S = O.adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, t)
        plain, m1, v1, _ = O.adamw_update(plain, g, m1, v1, S)
        th = O.reconstruct_weights(w16, ecc, "bf16", fmt_bits)
        th, m2, v2, _ = O.adamw_update(th, g, m2, v2, S)
        w16, ecc = O.split_weights(th, "bf16", fmt_bits)
    return plain, O.reconstruct_weights(w16, ecc, "bf16", fmt_bits)


def test_bf16_ecc16_reproduces_fp32_master_bitwise():
    plain, split = _run_ecc16_vs_plain(16)
    assert np.array_equal(plain.view(np.uint32), split.view(np.uint32))
    # and the 8-bit ECC does NOT (it is a 24-bit master), but stays close
    plain8, split8 = _run_ecc16_vs_plain(8)
    assert not np.array_equal(plain8, split8)
    # each step re-rounds the master to a 16-bit significand (8 + 8 bits)
    assert np.max(np.abs(plain8 - split8)) < 8 * 2 ** -16 * np.max(np.abs(plain8))


def test_full_step_tracks_unquantised():
    # sanity: the quantised step stays close to the unquantised trajectory
    rng = np.random.default_rng(24)
    n = 32 * 500 + 7
    x0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    st = fresh_adamw_state(x0)
    th = x0.copy(); m = np.zeros(n, np.float32); v = np.zeros(n, np.float32)
    hp = dict(HP)
    for t in range(1, 11):
        g = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
        gb = (g.astype(np.float32).view(np.uint32) + 0x8000 >> 16).astype(np.uint16)   # test-side bf16 cast
        gw = (gb.astype(np.uint32) << 16).view(np.float32)
        hp["step"] = t
        st = O.adamw_step(st, gb, hp)
        th, m, v, _ = O.adamw_update(th, gw, m, v, O.adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, t))
    q = O.reconstruct_weights(st["w16"], st["ecc"])
    # ten steps of ~lr each: parameters move ~1e-2 relative; quantised states
    # perturb the update by at most a few percent of that
    assert np.median(np.abs(q - th)) < 0.05 * 1e-3 * 10


def test_sgdm_full_step_first_step_equals_torch_buffer():
    rng = np.random.default_rng(25)
    x0 = (rng.standard_normal(64) * 0.02).astype(np.float32)
    st = fresh_sgdm_state(x0)
    g = (rng.standard_normal(64) * 1e-2).astype(np.float32)
    gb = (g.view(np.uint32) + 0x8000 >> 16).astype(np.uint16)
    gw = (gb.astype(np.uint32) << 16).view(np.float32)
    st2 = O.sgdm_step(st, gb, dict(lr=0.1, momentum=0.9, weight_decay=1e-4, step=1))
    th0 = O.reconstruct_weights(st["w16"], st["ecc"])
    d = gw + np.float32(1e-4) * th0
    want = th0 - np.float32(0.1) * d
    w16, ecc = O.split_weights(want)
    assert np.array_equal(st2["w16"], w16) and np.array_equal(st2["ecc"], ecc)


def test_bytes_per_param():
    # 16-bit weight + 8-bit ECC + 16-bit grad + 8-bit m + 8-bit v = 7 B/param,
    # plus one 16-bit scale per 32 elements for each of m and v: 7.125 B/param
    n = 32 * 1024
    st = fresh_adamw_state(np.zeros(n, np.float32))
    grad = np.zeros(n, np.uint16)
    total = sum(a.nbytes for a in st.values()) + grad.nbytes
    assert total / n == 7.125
    # the fp32 mixed-precision baseline: 4 master + 4 grad + 8 Adam = 16
    assert (4 + 4 + 8) == 16


def test_adam_l2_matches_torch_adam():
    # U6: coupled L2 decay added to the gradient (torch.optim.Adam weight_decay)
    rng = np.random.default_rng(30)
    x0 = (rng.standard_normal((7, 5)) * 0.02).astype(np.float32)
    grads = [(rng.standard_t(3, (7, 5)) * 1e-3).astype(np.float32) for _ in range(10)]
    p = torch.nn.Parameter(torch.tensor(x0, dtype=torch.float64))
    opt = torch.optim.Adam([p], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.1, foreach=False)
    th = x0.copy(); m = np.zeros_like(th); v = np.zeros_like(th)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        th, m, v, _ = O.adamw_update(th, g, m, v, O.adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.1, t, l2=True))
        ref = p.detach().numpy()
        assert np.max(np.abs(th - ref)) <= 1e-6 * np.max(np.abs(ref))
        assert np.max(np.abs((th - x0) - (ref - x0))) <= 1e-4 * np.max(np.abs(ref - x0))
    # and it differs from AdamW by far more than that (the decay is not decoupled)
    th2 = x0.copy(); m2 = np.zeros_like(th2); v2 = np.zeros_like(th2)
    for t, g in enumerate(grads, start=1):
        th2, m2, v2, _ = O.adamw_update(th2, g, m2, v2, O.adamw_scalars(1e-3, 0.9, 0.999, 1e-8, 0.1, t))
    assert np.max(np.abs(th2 - th)) > 1e-3 * np.max(np.abs(th - x0))


@pytest.mark.parametrize("nesterov,dampening", [(True, 0.0), (False, 0.5), (False, 0.0)])
def test_sgd_variants_match_torch(nesterov, dampening):
    rng = np.random.default_rng(31)
    x0 = (rng.standard_normal((7, 5)) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal((7, 5)) * 1e-2).astype(np.float32) for _ in range(10)]
    p = torch.nn.Parameter(torch.tensor(x0, dtype=torch.float64))
    opt = torch.optim.SGD([p], lr=0.1, momentum=0.9, weight_decay=1e-4, dampening=dampening,
                          nesterov=nesterov, foreach=False)
    S = O.sgdm_scalars(0.1, 0.9, 1e-4, dampening, nesterov)
    th = x0.copy(); b = np.zeros_like(th)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        th, b = O.sgdm_update(th, g, b, S, first=(t == 1))
        ref = p.detach().numpy()
        assert np.max(np.abs(th - ref)) <= 1e-6 * np.max(np.abs(ref))
        assert np.max(np.abs((th - x0) - (ref - x0))) <= 1e-4 * np.max(np.abs(ref - x0))


def test_adamw_quotient_is_one_division():
    # With beta1 = beta2 = 0, lr = 1, wd = 0 and theta = 0 the update reduces
    # to theta' = -RN32(g / RN32(|g| + eps)): m = g, v = g*g, sqrt(v) = |g|
    # (exact for a correctly rounded square of a float), step size 1.  The
    # quotient must be the exact rational g/d rounded once; the inputs are
    # kept where g * RN32(1/d) rounds to another float, so a reciprocal-
    # multiply (one rounding more) fails here.
    rng = np.random.default_rng(50)
    g = (rng.choice([-1, 1], 20000) * 10.0 ** rng.uniform(-3, 0, 20000)).astype(np.float32)
    eps = (10.0 ** rng.uniform(-4, 0, 20000)).astype(np.float32)
    d = (np.abs(g) + eps).astype(np.float32)
    recip = (g * (np.float32(1) / d)).astype(np.float32)
    div = (g / d).astype(np.float32)
    pick = np.nonzero(recip != div)[0][:300]
    assert pick.size >= 200
    for i in pick:
        S = O.adamw_scalars(1.0, 0.0, 0.0, float(eps[i]), 0.0, 1)
        assert S.step_size == 1 and S.ibc2 == 1 and S.decay == 1 and S.eps == eps[i]
        th, m, v, w = O.adamw_update(np.zeros(1, np.float32), g[i:i + 1], np.zeros(1, np.float32),
                                     np.zeros(1, np.float32), S)
        dd = rn32(abs(Fraction(float(g[i]))) + Fraction(float(eps[i])))
        want = -rn32(Fraction(float(g[i])) / dd)
        assert w[0] == abs(g[i])
        assert th[0] == f32(want), (float(g[i]), float(eps[i]), float(th[0]), float(want))


def test_adamw_update_rounds_once_per_operation():
    # The whole float32 sequence of the update (U3, and U6 for Adam) against
    # the same operations on exact rationals, each rounded once to binary32:
    # no contraction into fused multiply-adds, no wider intermediate, no
    # reordering.  Random moments, weights and hyperparameters.
    rng = np.random.default_rng(51)
    for trial in range(400):
        l2 = bool(trial % 3 == 0)
        hp = dict(lr=float(10 ** rng.uniform(-4, -1)), beta1=float(rng.uniform(0, 0.99)),
                  beta2=float(rng.uniform(0.9, 0.9999)), eps=float(10 ** rng.uniform(-9, -5)),
                  weight_decay=float(rng.uniform(0, 0.2)), step=int(rng.integers(1, 1000)))
        S = O.adamw_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"],
                            hp["step"], l2=l2)
        th0 = np.float32(rng.standard_normal() * 0.02)
        g0 = np.float32(rng.standard_t(3) * 1e-3)
        m0 = np.float32(rng.standard_t(3) * 1e-3)
        v0 = np.float32((rng.standard_t(3) * 1e-3) ** 2)
        th, m, v, w = O.adamw_update(np.array([th0]), np.array([g0]), np.array([m0]), np.array([v0]), S)
        F = lambda x: Fraction(float(x))
        T, G, M, V = F(th0), F(g0), F(m0), F(v0)
        if l2:
            G = rn32(G + rn32(F(S.wd) * T))
        M1 = rn32(rn32(F(S.b1) * M) + rn32(F(S.omb1) * G))
        V1 = rn32(rn32(F(S.b2) * V) + rn32(F(S.omb2) * rn32(G * G)))
        T1 = rn32(T * F(S.decay))
        W = rn32_sqrt(V1)
        D = rn32(rn32(W * F(S.ibc2)) + F(S.eps))
        T2 = rn32(T1 - rn32(F(S.step_size) * rn32(M1 / D)))
        assert (m[0], v[0], w[0], th[0]) == (f32(M1), f32(V1), f32(W), f32(T2)), (trial, hp)


def test_sgd_momentum0_ignores_dampening_like_torch():
    # U4: torch.optim.SGD with momentum 0 keeps no buffer, so dampening has no
    # effect; the oracle's buffer is then d at every step
    rng = np.random.default_rng(52)
    x0 = (rng.standard_normal((7, 5)) * 0.02).astype(np.float32)
    grads = [(rng.standard_normal((7, 5)) * 1e-2).astype(np.float32) for _ in range(6)]
    p = torch.nn.Parameter(torch.tensor(x0, dtype=torch.float64))
    opt = torch.optim.SGD([p], lr=0.1, momentum=0.0, weight_decay=1e-4, dampening=0.5, foreach=False)
    S = O.sgdm_scalars(0.1, 0.0, 1e-4, 0.5)
    th = x0.copy(); b = np.zeros_like(th)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        th, b = O.sgdm_update(th, g, b, S, first=O.sgdm_first(t, 0.0))
        ref = p.detach().numpy()
        assert np.max(np.abs(th - ref)) <= 1e-6 * np.max(np.abs(ref))
        assert np.max(np.abs((th - x0) - (ref - x0))) <= 1e-4 * np.max(np.abs(ref - x0))
    # the fused step: every step is theta - lr*d, split again
    st = fresh_sgdm_state(x0.ravel())
    for t, g in enumerate(grads, start=1):
        gb = (g.ravel().view(np.uint32) + 0x8000 >> 16).astype(np.uint16)
        gw = (gb.astype(np.uint32) << 16).view(np.float32)
        th0 = O.reconstruct_weights(st["w16"], st["ecc"])
        st = O.sgdm_step(st, gb, dict(lr=0.1, momentum=0.0, weight_decay=1e-4, dampening=0.5, step=t))
        want = th0 - np.float32(0.1) * (gw + np.float32(1e-4) * th0)
        w16, ecc = O.split_weights(want)
        assert np.array_equal(st["w16"], w16) and np.array_equal(st["ecc"], ecc)


@pytest.mark.parametrize("fmt,ecc_bits,codec", [("bf16", 8, "companded"), ("bf16", 16, "linear"),
                                                ("fp16", 8, "companded")])
def test_adamw_step_first_step_closed_form(fmt, ecc_bits, codec):
    # The composition of adamw_step, pinned at step 1 from fresh states: the
    # zero codes and scales decode to m = v = 0, so the new moments are
    # m1 = RN((1-b1)*g), v1 = RN((1-b2)*RN(g*g)) and the new master is
    # RN(RN(th*decay) - RN(step_size*RN(m1/d))), d = RN(RN(sqrt(v1)*ibc2) + eps),
    # computed here on exact rationals.  The step must then hold exactly the
    # split of that master and the block scales and codes of m1 and v1 (a
    # wiring mistake -- old moments encoded, scales swapped, v's scale taken
    # from v instead of its root, the split fed the pre-update master -- fails).
    rng = np.random.default_rng(61)
    n = 101                                            # three full blocks and a ragged one
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g32 = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
    if fmt == "fp16":
        gb = g32.astype(np.float16).view(np.uint16)
    else:
        gb = torch.tensor(g32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    st = fresh_adamw_state(x, fmt, ecc_bits)
    out = O.adamw_step(st, gb, hp, fmt, ecc_bits, codec)
    S = O.adamw_scalars(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], hp["step"])
    theta0 = O.reconstruct_weights(st["w16"], st["ecc"], fmt, ecc_bits)
    g = (gb.view(np.float16).astype(np.float32) if fmt == "fp16"
         else (gb.astype(np.uint32) << 16).view(np.float32))          # exact widening
    F = lambda v: Fraction(float(v))
    m1 = np.empty(n, np.float32); v1 = np.empty(n, np.float32); th1 = np.empty(n, np.float32)
    for i in range(n):
        G = F(g[i])
        M = rn32(F(S.omb1) * G)
        V = rn32(F(S.omb2) * rn32(G * G))
        D = rn32(rn32(rn32_sqrt(V) * F(S.ibc2)) + F(S.eps))
        T = rn32(rn32(F(theta0[i]) * F(S.decay)) - rn32(F(S.step_size) * rn32(M / D)))
        m1[i], v1[i], th1[i] = f32(M), f32(V), f32(T)
    w_want, e_want = O.split_weights(th1, fmt, ecc_bits)
    ms, vs = O.block_scales(m1, "m"), O.block_scales(v1, "v")
    assert np.array_equal(out["w16"], w_want) and np.array_equal(out["ecc"], e_want)
    assert np.array_equal(out["m_s"], ms) and np.array_equal(out["v_s"], vs)
    assert np.array_equal(out["m_q"], O.encode_momentum(m1, ms, codec))
    assert np.array_equal(out["v_q"], O.encode_variance(v1, vs, codec))
    assert np.count_nonzero(out["m_q"]) > n // 2 and np.count_nonzero(out["v_q"]) > n // 2


@pytest.mark.parametrize("nesterov,codec", [(False, "companded"), (True, "linear")])
def test_sgdm_step_first_step_closed_form(nesterov, codec):
    # The composition of sgdm_step at step 1 (U4): the buffer is set to
    # d = RN(g + RN(wd*th)) whatever the stored codes hold, and the master
    # moves by RN(lr*u), u = d (plain) or RN(d + RN(mu*d)) (Nesterov); on
    # exact rationals here.  The step must hold exactly the split of that
    # master and the block scales and codes of d.  Stored codes are random
    # to show step 1 ignores them.
    rng = np.random.default_rng(62)
    n = 77
    x = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g32 = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    gb = torch.tensor(g32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    st = fresh_sgdm_state(x)
    st["b_q"] = rng.integers(-127, 128, n).astype(np.int8)
    st["b_s"] = np.full(-(-n // 32), 0x3C00, np.uint16)            # scale 1.0
    hp = dict(lr=0.1, momentum=0.9, weight_decay=1e-4, dampening=0.0, nesterov=nesterov, step=1)
    out = O.sgdm_step(st, gb, hp, "bf16", 8, codec)
    S = O.sgdm_scalars(hp["lr"], hp["momentum"], hp["weight_decay"], 0.0, nesterov)
    theta0 = O.reconstruct_weights(st["w16"], st["ecc"], "bf16", 8)
    g = (gb.astype(np.uint32) << 16).view(np.float32)                  # exact widening
    F = lambda v: Fraction(float(v))
    d1 = np.empty(n, np.float32); th1 = np.empty(n, np.float32)
    for i in range(n):
        T = F(theta0[i])
        D = rn32(F(g[i]) + rn32(F(S.wd) * T))
        U = rn32(D + rn32(F(S.mu) * D)) if nesterov else D
        d1[i], th1[i] = f32(D), f32(rn32(T - rn32(F(S.lr) * U)))
    w_want, e_want = O.split_weights(th1, "bf16", 8)
    bs = O.block_scales(d1, "m")
    assert np.array_equal(out["w16"], w_want) and np.array_equal(out["ecc"], e_want)
    assert np.array_equal(out["b_s"], bs)
    assert np.array_equal(out["b_q"], O.encode_momentum(d1, bs, codec))
