"""Checks that pin the fp64 oracle to facts that do not come from the oracle.

Each check takes an oracle object (with ``fwd`` and ``bwd`` methods, see
``oracle.OracleLib``) and returns the largest discrepancy it found.  The pin
tests call them with the real oracle and require tiny errors; the mutation
test calls them with deliberately broken builds of the oracle source and
requires that at least one check notices.

What each check compares against (none of it re-types the recurrence):

* ``t1_closed_form``   -- one token in matrix form, h1 = h0 diag(w) + v k^T
                          + (h0 a) b^T and y = h1 r, with numpy matmuls.
* ``linear_attention`` -- w = 1, a = b = 0 turns the state into a running sum
                          of v k^T, so y is causal linear attention
                          tril(R K^T) V plus the h0 readout (RWKV as an RNN
                          that trains like a parallel model: RWKV-LM pages).
* ``decay_scan``       -- a = 0 leaves a per-channel decayed sum with the
                          explicit product form of the decays; db must be 0.
* ``delta_rule``       -- w = 1, a = -k, b = k for a unit k gives the delta
                          rule, whose state maps k_t to v_t exactly, so r = k
                          reads v back (the "model trained one step per token"
                          view of the RWKV-7 news page).
* ``split_sequence``   -- running T1 tokens then T2 tokens with the state
                          handed over equals running T1+T2 tokens (the RNN
                          state-passing usage of the RWKV-LM README page), and
                          every checkpoint equals the state after 32c tokens.
* ``finite_difference``-- central differences of the (pinned) forward against
                          every gradient the backward returns, tiny shapes.
* ``adjoint``          -- <grad, delta> against a directional difference at
                          a larger shape.
* ``autograd``         -- torch.autograd through a naive fp64 forward loop.

The time-mix prologue (w, a, b from raw projections):

* ``proj_identities``  -- facts of the logistic function and of a unit
                          vector, not its formula: w(x) w(-x) = exp(-e^-1/2)
                          and w(0)^2 equals it too; w decreases in w_raw and
                          tends to 1 and exp(-e^-1/2); a has unit norm and
                          points against kappa; a, b do not change when kappa
                          is scaled; the gate b / (-a) does not depend on
                          kappa, is 1/2 at alpha = 0 and g(x) + g(-x) = 1;
                          kappa = 0 gives a = b = 0.
* ``proj_finite_difference`` -- central differences of the (pinned) prologue
                          against its backward, and the gradient w.r.t. kappa
                          orthogonal to kappa (scale invariance).
* ``proj_composed``    -- central differences of the whole layer (prologue,
                          then the recurrence) against the chain of the two
                          backwards, at a tiny shape.
* ``proj_recipe``      -- the prologue applied to the raw draws of the input
                          generator gives the w, a, b that the generator's own
                          fp32 recipe forms from the same draws (an
                          independent implementation, in torch).
"""
from __future__ import annotations

import numpy as np
import torch


def rand_inputs(rng, B, T, H, D, w_lo=0.5, h0=True, kscale=0.5):
    r = rng.standard_normal((B, T, H, D))
    w = rng.uniform(w_lo, 1.0, (B, T, H, D))
    k = rng.standard_normal((B, T, H, D)) * kscale
    v = rng.standard_normal((B, T, H, D))
    kap = rng.standard_normal((B, T, H, D))
    kap /= np.linalg.norm(kap, axis=-1, keepdims=True)
    a = -kap
    b = kap * rng.uniform(0.0, 1.0, (B, T, H, 1))
    # make a and b not parallel so that swapping their roles is visible
    b = b + 0.3 * rng.standard_normal((B, T, H, D)) / np.sqrt(D)
    h0v = rng.standard_normal((B, H, D, D)) * 0.3 if h0 else None
    return r, w, k, v, a, b, h0v


def rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def t1_closed_form(orc, seed=1):
    rng = np.random.default_rng(seed)
    B, H, D = 2, 3, 16
    r, w, k, v, a, b, h0 = rand_inputs(rng, B, 1, H, D)
    y, ck, hT = orc.fwd(r, w, k, v, a, b, h0)
    err = 0.0
    for bb in range(B):
        for hh in range(H):
            S0 = h0[bb, hh]
            wt, kt, vt, at, bt, rt = (x[bb, 0, hh] for x in (w, k, v, a, b, r))
            S1 = S0 @ np.diag(wt) + np.outer(vt, kt) + np.outer(S0 @ at, bt)
            err = max(err, rel(hT[bb, hh], S1), rel(y[bb, 0, hh], S1 @ rt),
                      rel(ck[bb, hh, 0], S0))
    return err


def linear_attention(orc, seed=2):
    rng = np.random.default_rng(seed)
    B, T, H, D = 2, 45, 2, 16
    r, _, k, v, _, _, h0 = rand_inputs(rng, B, T, H, D)
    w = np.ones_like(r)
    zero = np.zeros_like(r)
    y, _, hT = orc.fwd(r, w, k, v, zero, zero, h0)
    err = 0.0
    for bb in range(B):
        for hh in range(H):
            R, K, V = r[bb, :, hh], k[bb, :, hh], v[bb, :, hh]
            Y = np.tril(R @ K.T) @ V + R @ h0[bb, hh].T
            S = h0[bb, hh] + V.T @ K
            err = max(err, rel(y[bb, :, hh], Y), rel(hT[bb, hh], S))
    return err


def decay_scan(orc, seed=3):
    rng = np.random.default_rng(seed)
    B, T, H, D = 1, 23, 2, 12
    r, w, k, v, _, b, h0 = rand_inputs(rng, B, T, H, D)
    a = np.zeros_like(r)
    y, _, hT = orc.fwd(r, w, k, v, a, b, h0)
    err = 0.0
    for hh in range(H):
        W, K, V, R = w[0, :, hh], k[0, :, hh], v[0, :, hh], r[0, :, hh]
        for t in range(T):
            yt = np.zeros(D)
            for s in range(t + 1):
                dec = np.prod(W[s + 1:t + 1], axis=0)          # prod_{u=s+1..t} w_u
                yt += V[s] * np.dot(K[s] * dec, R[t])
            dec0 = np.prod(W[:t + 1], axis=0)                 # prod_{u<=t} w_u
            yt += h0[0, hh] @ (dec0 * R[t])
            err = max(err, rel(y[0, t, hh], yt))
    dy = rng.standard_normal(r.shape)
    grads = orc.bwd(r, w, k, v, a, b, dy, h0, rng.standard_normal(h0.shape))
    err = max(err, float(np.abs(grads[5]).max()))            # db must vanish exactly
    return err


def delta_rule(orc, seed=4):
    rng = np.random.default_rng(seed)
    B, T, H, D = 2, 40, 2, 16
    kh = rng.standard_normal((B, T, H, D))
    kh /= np.linalg.norm(kh, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, D))
    h0 = rng.standard_normal((B, H, D, D))
    ones = np.ones_like(kh)
    y, _, hT = orc.fwd(kh, ones, kh, v, -kh, kh, h0)
    # after the last token the state maps its key onto its value
    err = rel(y, v)
    for bb in range(B):
        for hh in range(H):
            err = max(err, rel(hT[bb, hh] @ kh[bb, -1, hh], v[bb, -1, hh]))
    return err


def split_sequence(orc, seed=5):
    rng = np.random.default_rng(seed)
    B, T, H, D = 1, 100, 2, 8
    r, w, k, v, a, b, h0 = rand_inputs(rng, B, T, H, D)
    y, ck, hT = orc.fwd(r, w, k, v, a, b, h0)
    T1 = 37
    s1 = lambda x: x[:, :T1]
    s2 = lambda x: x[:, T1:]
    y1, _, h1 = orc.fwd(*map(s1, (r, w, k, v, a, b)), h0)
    y2, _, h2 = orc.fwd(*map(s2, (r, w, k, v, a, b)), h1)
    err = max(rel(np.concatenate([y1, y2], axis=1), y), rel(h2, hT))
    for c in range(ck.shape[2]):
        if c == 0:
            ref = h0
        else:
            ref = orc.fwd(*(x[:, :32 * c] for x in (r, w, k, v, a, b)), h0)[2]
        err = max(err, rel(ck[:, :, c], ref))
    return err


def _loss(orc, ins, h0, dy, dhT):
    y, _, hT = orc.fwd(*ins, h0, want_ckpt=False)
    return float(np.sum(y * dy) + np.sum(hT * dhT))


def finite_difference(orc, seed=6, T=7, D=5):
    rng = np.random.default_rng(seed)
    B, H = 1, 1
    r, w, k, v, a, b, h0 = rand_inputs(rng, B, T, H, D)
    ins = [r, w, k, v, a, b]
    dy = rng.standard_normal(r.shape)
    dhT = rng.standard_normal(h0.shape)
    grads = orc.bwd(*ins, dy, h0, dhT)
    eps = 1e-6
    err = 0.0
    for n in range(6):
        g = grads[n]
        num = np.zeros_like(g)
        for idx in np.ndindex(*g.shape):
            p = [x.copy() for x in ins]
            p[n][idx] += eps
            m = [x.copy() for x in ins]
            m[n][idx] -= eps
            num[idx] = (_loss(orc, p, h0, dy, dhT) - _loss(orc, m, h0, dy, dhT)) / (2 * eps)
        err = max(err, rel(g, num))
    num = np.zeros_like(h0)
    for idx in np.ndindex(*h0.shape):
        p = h0.copy()
        p[idx] += eps
        m = h0.copy()
        m[idx] -= eps
        num[idx] = (_loss(orc, ins, p, dy, dhT) - _loss(orc, ins, m, dy, dhT)) / (2 * eps)
    err = max(err, rel(grads[6], num))
    return err


def adjoint(orc, seed=7):
    rng = np.random.default_rng(seed)
    B, T, H, D = 2, 70, 2, 16
    r, w, k, v, a, b, h0 = rand_inputs(rng, B, T, H, D)
    ins = [r, w, k, v, a, b, h0]
    dy = rng.standard_normal(r.shape)
    dhT = rng.standard_normal(h0.shape)
    grads = orc.bwd(*ins[:6], dy, h0, dhT)
    err = 0.0
    eps = 1e-6
    for n in range(7):
        d = rng.standard_normal(ins[n].shape)
        p = [x.copy() for x in ins]
        p[n] = p[n] + eps * d
        m = [x.copy() for x in ins]
        m[n] = m[n] - eps * d
        fd = (_loss(orc, p[:6], p[6], dy, dhT) - _loss(orc, m[:6], m[6], dy, dhT)) / (2 * eps)
        an = float(np.sum(grads[n] * d))
        err = max(err, abs(fd - an) / max(1.0, abs(an)))
    return err


def autograd(orc, seed=8):
    rng = np.random.default_rng(seed)
    B, T, H, D = 2, 9, 2, 5
    r, w, k, v, a, b, h0 = rand_inputs(rng, B, T, H, D)
    dy = rng.standard_normal(r.shape)
    dhT = rng.standard_normal(h0.shape)
    tin = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (r, w, k, v, a, b, h0)]
    tr, tw, tk, tv, ta, tb, th = tin
    ys = []
    hs = []
    for bb in range(B):
        for hh in range(H):
            S = th[bb, hh]
            yrow = []
            for t in range(T):
                sa = S @ ta[bb, t, hh]
                S = S * tw[bb, t, hh][None, :] + torch.outer(tv[bb, t, hh], tk[bb, t, hh]) \
                    + torch.outer(sa, tb[bb, t, hh])
                yrow.append(S @ tr[bb, t, hh])
            ys.append(torch.stack(yrow))
            hs.append(S)
    Y = torch.stack(ys).reshape(B, H, T, D).permute(0, 2, 1, 3)
    HT = torch.stack(hs).reshape(B, H, D, D)
    L = (Y * torch.tensor(dy)).sum() + (HT * torch.tensor(dhT)).sum()
    L.backward()
    grads = orc.bwd(r, w, k, v, a, b, dy, h0, dhT)
    y, _, hT = orc.fwd(r, w, k, v, a, b, h0)
    err = max(rel(y, Y.detach().numpy()), rel(hT, HT.detach().numpy()))
    for n in range(7):
        err = max(err, rel(grads[n], tin[n].grad.numpy()))
    return err


def proj_identities(orc, seed=9):
    rng = np.random.default_rng(seed)
    D = 8
    x = rng.standard_normal((4, D)) * 3
    kap = rng.standard_normal((4, D))
    al = rng.standard_normal((4, D)) * 2
    wp, ap, bp = orc.proj_fwd(x, kap, al)
    wm, _, _ = orc.proj_fwd(-x, kap, al)
    lim = np.exp(-np.exp(-0.5))
    err = float(np.max(np.abs(wp * wm - lim)))
    w0, _, _ = orc.proj_fwd(np.zeros((1, D)), kap[:1], al[:1])
    err = max(err, float(np.max(np.abs(w0 * w0 - lim))))
    ws, _, _ = orc.proj_fwd(np.linspace(-40, 40, D)[None, :], kap[:1], al[:1])
    err = max(err, abs(ws[0, 0] - 1.0), abs(ws[0, -1] - lim))
    if not np.all(np.diff(ws[0]) < 0):
        err = max(err, 1.0)
    err = max(err, float(np.max(np.abs(np.linalg.norm(ap, axis=-1) - 1.0))))
    err = max(err, float(np.max(np.abs(np.sum(ap * kap, axis=-1) + np.linalg.norm(kap, axis=-1)))))
    _, a3, b3 = orc.proj_fwd(x, 3.0 * kap, al)
    err = max(err, float(np.max(np.abs(a3 - ap))), float(np.max(np.abs(b3 - bp))))
    kap2 = rng.standard_normal((4, D))
    _, a2, b2 = orc.proj_fwd(x, kap2, al)
    gate, gate2 = bp / -ap, b2 / -a2
    err = max(err, float(np.max(np.abs(gate - gate2))))
    _, am, bm = orc.proj_fwd(x, kap, -al)
    err = max(err, float(np.max(np.abs(gate + bm / -am - 1.0))))
    _, ah, bh = orc.proj_fwd(x, kap, np.zeros_like(al))
    err = max(err, float(np.max(np.abs(bh / -ah - 0.5))))
    _, az, bz = orc.proj_fwd(x[:1], np.zeros((1, D)), al[:1])
    err = max(err, float(np.max(np.abs(az))), float(np.max(np.abs(bz))))
    return err


def _proj_loss(orc, raws, cw, ca, cb):
    w, a, b = orc.proj_fwd(*raws)
    return float(np.sum(w * cw) + np.sum(a * ca) + np.sum(b * cb))


def proj_finite_difference(orc, seed=10):
    rng = np.random.default_rng(seed)
    shape = (3, 6)
    raws = [rng.standard_normal(shape) * s for s in (2.0, 1.0, 2.0)]
    cw, ca, cb = (rng.standard_normal(shape) for _ in range(3))
    grads = orc.proj_bwd(*raws, cw, ca, cb)
    eps = 1e-6
    err = 0.0
    for n in range(3):
        num = np.zeros(shape)
        for idx in np.ndindex(*shape):
            p = [x.copy() for x in raws]
            p[n][idx] += eps
            m = [x.copy() for x in raws]
            m[n][idx] -= eps
            num[idx] = (_proj_loss(orc, p, cw, ca, cb) - _proj_loss(orc, m, cw, ca, cb)) / (2 * eps)
        err = max(err, rel(grads[n], num))
    # a and b depend on kappa only through its direction
    err = max(err, float(np.max(np.abs(np.sum(grads[1] * raws[1], axis=-1)))))
    return err


def proj_composed(orc, seed=11):
    rng = np.random.default_rng(seed)
    B, T, H, D = 1, 5, 1, 6
    r = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D)) * 0.5
    v = rng.standard_normal((B, T, H, D))
    raws = [rng.standard_normal((B, T, H, D)) for _ in range(3)]
    h0 = rng.standard_normal((B, H, D, D)) * 0.3
    dy = rng.standard_normal((B, T, H, D))
    dhT = rng.standard_normal((B, H, D, D))

    def loss(rw):
        w, a, b = orc.proj_fwd(*rw)
        return _loss(orc, [r, w, k, v, a, b], h0, dy, dhT)

    w, a, b = orc.proj_fwd(*raws)
    g = orc.bwd(r, w, k, v, a, b, dy, h0, dhT)
    chain = orc.proj_bwd(*raws, g[1], g[4], g[5])
    eps = 1e-6
    err = 0.0
    for n in range(3):
        num = np.zeros(raws[n].shape)
        for idx in np.ndindex(*raws[n].shape):
            p = [x.copy() for x in raws]
            p[n][idx] += eps
            m = [x.copy() for x in raws]
            m[n][idx] -= eps
            num[idx] = (loss(p) - loss(m)) / (2 * eps)
        err = max(err, rel(chain[n], num))
    return err


def proj_recipe(orc, seed=12):
    from linear_rnn_lm_amd.inputs import make_inputs, make_proj_inputs
    x = make_inputs(2, 40, 3, torch.float32, seed=seed)
    xr = make_proj_inputs(2, 40, 3, torch.float32, seed=seed)
    err = max(rel(xr.r.numpy(), x.r.numpy()), rel(xr.k.numpy(), x.k.numpy()), rel(xr.v.numpy(), x.v.numpy()))
    w, a, b = orc.proj_fwd(xr.w_raw, xr.kappa, xr.alpha)
    return max(err, rel(w, x.w.numpy()), rel(a, x.a.numpy()), rel(b, x.b.numpy()))


ALL = {
    "t1_closed_form": t1_closed_form,
    "linear_attention": linear_attention,
    "decay_scan": decay_scan,
    "delta_rule": delta_rule,
    "split_sequence": split_sequence,
    "finite_difference": finite_difference,
    "adjoint": adjoint,
    "autograd": autograd,
    "proj_identities": proj_identities,
    "proj_finite_difference": proj_finite_difference,
    "proj_composed": proj_composed,
    "proj_recipe": proj_recipe,
}

# tolerance of each check for a correct fp64 oracle
TOL = {
    "t1_closed_form": 1e-13,
    "linear_attention": 1e-12,
    "decay_scan": 1e-12,
    "delta_rule": 1e-12,
    "split_sequence": 1e-13,
    "finite_difference": 1e-7,
    "adjoint": 1e-6,
    "autograd": 1e-12,
    "proj_identities": 1e-14,
    "proj_finite_difference": 1e-7,
    "proj_composed": 1e-7,
    "proj_recipe": 1e-6,
}
