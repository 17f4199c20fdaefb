"""Pins of the oracle's backward pass (oracle.bptt) against things other than itself (CPU).

* central finite differences of the forward oracle's loss, entry by entry, for every
  parameter tensor and the encoder outputs (the derivative from its definition);
* torch autograd through a forward written here with torch operations (every entry);
* invariants: feedback scale zero cuts the start state out of every gradient; encoder
  outputs after the last token that carries loss get exactly zero gradient; the gradient is
  linear in the upstream gradient;
* truncation: the truncated gradients equal finite differences of a forward in which the
  detached tensors are frozen at their values at every segment start; detaching the state
  alone leaves the window path open.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import RLTConfig, make_encoder_outputs, make_params


def tiny(**kw):
    base = dict(name="bwd", d=16, n_heads=2, head_dim=8, n_layers=2, ffn=24, window=3,
                n_groups=2, alpha=0.7, batch=2, seq_len=6, dtype="fp32", sigma=0.3)
    base.update(kw)
    return RLTConfig(**base)


def setup(cfg, seed=0):
    p = make_params(cfg, seed=seed, random_gains=True, random_gate_bias=True)
    p = {k: np.asarray(v, np.float64) for k, v in p.items()}
    e = make_encoder_outputs(cfg, range(cfg.batch), seed=seed).astype(np.float64)
    G = np.random.default_rng(seed + 100).standard_normal(e.shape)
    return p, e, G


def loss_of(p, cfg, e, G):
    traj, _ = oracle.run_sequence(p, cfg, e)
    return oracle.sequence_loss(traj, G)


CASES = [
    dict(),                                         # G = L, window shorter than the sequence
    dict(n_groups=1, alpha=1.0, window=2),          # shared memory, full feedback
    dict(window=1, n_layers=1),                     # no retained entries
    dict(window=9, n_heads=4, head_dim=4),          # window longer than the sequence
]


@pytest.mark.parametrize("case", CASES)
def test_bptt_matches_finite_differences(case):
    cfg = tiny(**case)
    p, e, G = setup(cfg, seed=len(case))
    traj, gr, de = oracle.bptt(p, cfg, e, G)
    ref, _ = oracle.run_sequence(p, cfg, e)
    assert np.array_equal(traj, ref)
    rng = np.random.default_rng(11)
    h = 1e-5
    for name in oracle.GRAD_NAMES:
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in p[name].shape)
            pp = {k: v.copy() for k, v in p.items()}
            pp[name][idx] += h
            lp = loss_of(pp, cfg, e, G)
            pp[name][idx] -= 2 * h
            lm = loss_of(pp, cfg, e, G)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - gr[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, gr[name][idx])
    for _ in range(8):
        idx = tuple(int(rng.integers(0, s)) for s in e.shape)
        ee = e.copy()
        ee[idx] += h
        lp = loss_of(p, cfg, ee, G)
        ee[idx] -= 2 * h
        lm = loss_of(p, cfg, ee, G)
        fd = (lp - lm) / (2 * h)
        assert abs(fd - de[idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, de[idx])


# --- torch autograd through a forward written with torch operations -----------------------

def torch_forward(tp, cfg, e):
    """The decoder over e [B, n, d] from s*, written with torch ops for autograd."""
    B, n, d = e.shape
    H, hd, L, W = cfg.n_heads, cfg.head_dim, cfg.n_layers, cfg.window

    def norm(x, gain):
        return gain * x * torch.rsqrt((x * x).mean(-1, keepdim=True) + cfg.eps)

    def attn(q, keys, vals):  # q [B, d]; keys, vals [B, m, d]
        m = keys.shape[1]
        qh = q.view(B, H, 1, hd)
        kh = keys.view(B, m, H, hd).transpose(1, 2)
        vh = vals.view(B, m, H, hd).transpose(1, 2)
        w = torch.softmax((qh * kh).sum(-1) / hd ** 0.5, dim=-1)  # [B, H, m]
        return (w.unsqueeze(-1) * vh).sum(2).reshape(B, d)

    mk = [e @ tp["wmk"][g] for g in range(tp["wmk"].shape[0])]
    mv = [e @ tp["wmv"][g] for g in range(tp["wmv"].shape[0])]
    s = tp["s_star"].expand(B, d)
    ks = [[] for _ in range(L)]
    vs = [[] for _ in range(L)]
    out = []
    for t in range(n):
        u = cfg.alpha * s
        g = torch.sigmoid(torch.cat([e[:, t], u], -1) @ tp["w_gate"] + tp["b_gate"])
        h = g * e[:, t] + (1 - g) * u
        for l in range(L):
            gm = 0 if cfg.n_groups == 1 else l
            a = norm(h, tp["gamma"][l, 0])
            ks[l].append(a @ tp["wk"][l])
            vs[l].append(a @ tp["wv"][l])
            lo = max(0, t - W + 1)
            h = h + attn(a @ tp["wq"][l], torch.stack(ks[l][lo:], 1),
                         torch.stack(vs[l][lo:], 1)) @ tp["wo"][l]
            c = norm(h, tp["gamma"][l, 1])
            h = h + attn(c @ tp["wcq"][l], mk[gm][:, :t + 1], mv[gm][:, :t + 1]) @ tp["wco"][l]
            f = norm(h, tp["gamma"][l, 2])
            h = h + (torch.nn.functional.silu(f @ tp["w1"][l]) * (f @ tp["w3"][l])) @ tp["w2"][l]
        s = h
        out.append(s)
    return torch.stack(out, 1)


@pytest.mark.parametrize("case", [dict(), dict(n_groups=1, alpha=1.0, window=4, seq_len=9)])
def test_bptt_matches_torch_autograd(case):
    cfg = tiny(**case)
    p, e, G = setup(cfg, seed=3)
    traj, gr, de = oracle.bptt(p, cfg, e, G)
    tp = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in p.items()}
    te = torch.tensor(e, requires_grad=True)
    ttraj = torch_forward(tp, cfg, te)
    assert np.allclose(ttraj.detach().numpy(), traj, rtol=0, atol=1e-12)
    (ttraj * torch.tensor(G)).sum().backward()
    for name in oracle.GRAD_NAMES:
        ref = tp[name].grad.numpy()
        np.testing.assert_allclose(gr[name], ref, rtol=1e-9, atol=1e-11, err_msg=name)
    np.testing.assert_allclose(de, te.grad.numpy(), rtol=1e-9, atol=1e-11)


# --- invariants ---------------------------------------------------------------------------

def test_feedback_zero_cuts_the_start_state():
    cfg = tiny(alpha=0.0)
    p, e, G = setup(cfg, seed=7)
    _, gr, _ = oracle.bptt(p, cfg, e, G)
    assert not np.any(gr["s_star"])
    p2 = dict(p)
    p2["s_star"] = np.random.default_rng(1).standard_normal(cfg.d)
    _, gr2, _ = oracle.bptt(p2, cfg, e, G)
    for name in oracle.GRAD_NAMES:
        assert np.array_equal(gr[name], gr2[name]), name


def test_later_encoder_outputs_get_no_gradient():
    cfg = tiny(seq_len=7)
    p, e, G = setup(cfg, seed=8)
    G[:, 4:] = 0.0  # loss on s_1 .. s_4 only
    _, _, de = oracle.bptt(p, cfg, e, G)
    assert not np.any(de[:, 4:])
    assert np.all(np.linalg.norm(de[:, :4], axis=-1) > 0)


def test_gradient_is_linear_in_the_upstream_gradient():
    cfg = tiny()
    p, e, G1 = setup(cfg, seed=9)
    G2 = np.random.default_rng(4).standard_normal(e.shape)
    _, a, da = oracle.bptt(p, cfg, e, G1)
    _, b, db = oracle.bptt(p, cfg, e, G2)
    _, c, dc = oracle.bptt(p, cfg, e, 2.0 * G1 - G2)
    for name in oracle.GRAD_NAMES:
        np.testing.assert_allclose(c[name], 2.0 * a[name] - b[name], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dc, 2.0 * da - db, rtol=1e-9, atol=1e-12)


# --- truncation: every detached tensor named -----------------------------------------------

def frozen_forward_loss(p, cfg, e, G, seg, detach, base):
    """The loss of a forward in which, at every segment start, the detached tensors are
    replaced by their values in the unperturbed run (`base`: state before each segment start),
    so they enter the segment as constants; the memory is recomputed from p and e."""
    km, vm = oracle.memory_projection(p, e)
    st = oracle.init_state(p, cfg, e.shape[0])
    loss = 0.0
    for t in range(e.shape[1]):
        if t > 0 and t % seg == 0:
            s0, ck, cv = base[t]
            if "state" in detach:
                st.s = s0.copy()
            if "window" in detach:
                st.cache_k = [list(x) for x in ck]
                st.cache_v = [list(x) for x in cv]
        s_t = oracle.decoder_step(p, cfg, st, km, vm, e[:, t])
        loss += float(np.sum(G[:, t] * s_t))
    return loss


def base_states(p, cfg, e, seg):
    km, vm = oracle.memory_projection(p, e)
    st = oracle.init_state(p, cfg, e.shape[0])
    out = {}
    for t in range(e.shape[1]):
        if t > 0 and t % seg == 0:
            out[t] = (st.s.copy(), [list(x) for x in st.cache_k], [list(x) for x in st.cache_v])
        oracle.decoder_step(p, cfg, st, km, vm, e[:, t])
    return out


@pytest.mark.parametrize("detach", [("state",), ("window",), ("state", "window")])
def test_truncated_bptt_matches_finite_differences_of_the_frozen_forward(detach):
    cfg = tiny(window=3, seq_len=8)
    p, e, G = setup(cfg, seed=13)
    seg = 3
    _, gr, de = oracle.bptt(p, cfg, e, G, segment=seg, detach=detach)
    base = base_states(p, cfg, e, seg)
    rng = np.random.default_rng(17)
    h = 1e-5
    checks = [(name, tuple(int(rng.integers(0, s)) for s in p[name].shape))
              for name in oracle.GRAD_NAMES for _ in range(2)]
    for name, idx in checks:
        pp = {k: v.copy() for k, v in p.items()}
        pp[name][idx] += h
        lp = frozen_forward_loss(pp, cfg, e, G, seg, detach, base)
        pp[name][idx] -= 2 * h
        lm = frozen_forward_loss(pp, cfg, e, G, seg, detach, base)
        fd = (lp - lm) / (2 * h)
        assert abs(fd - gr[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, gr[name][idx])
    for _ in range(6):
        idx = tuple(int(rng.integers(0, s)) for s in e.shape)
        ee = e.copy()
        ee[idx] += h
        lp = frozen_forward_loss(p, cfg, ee, G, seg, detach, base)
        ee[idx] -= 2 * h
        lm = frozen_forward_loss(p, cfg, ee, G, seg, detach, base)
        assert abs((lp - lm) / (2 * h) - de[idx]) <= 1e-6 * max(1.0, abs(de[idx])), idx


def test_detaching_the_state_alone_leaves_the_window_path_open():
    """The trap named on the first page: with no memory path (zero memory projections) and loss
    only on the second segment, detaching s still lets gradient into the first segment through
    the window's keys/values of its last W - 1 tokens, and from there, along the first segment's
    own (undetached) state, to every token of it; detaching s and the window cuts it."""
    cfg = tiny(window=3, seq_len=8)
    p, e, G = setup(cfg, seed=19)
    p["wmk"][:] = 0.0
    p["wmv"][:] = 0.0
    seg = 4
    G[:, :seg] = 0.0
    _, _, de_full = oracle.bptt(p, cfg, e, G)
    _, _, de_s = oracle.bptt(p, cfg, e, G, segment=seg, detach=("state",))
    _, _, de_sw = oracle.bptt(p, cfg, e, G, segment=seg, detach=("state", "window"))
    first = np.linalg.norm(de_full[:, :seg], axis=-1)
    assert np.all(first > 0)
    leak = np.linalg.norm(de_s[:, :seg], axis=-1)
    assert np.all(leak > 0)
    assert not np.any(de_sw[:, :seg])
    np.testing.assert_allclose(de_sw[:, seg:], de_s[:, seg:], rtol=1e-12, atol=1e-14)
