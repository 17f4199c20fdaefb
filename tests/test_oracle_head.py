"""Pins of the encoder and readout/sampler oracle (oracle/rlt_head.py), none of which re-types
the oracle: library routines (torch's causal scaled-dot-product attention, rms_norm, silu,
log_softmax), closed forms, invariants, a hand-worked fixture and the exact distribution of
the inverse-CDF draw on a grid of uniforms."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import RLTConfig, make_head_params, make_params, make_tokens

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sampler_v4.json")


def cfg_small(**kw):
    base = dict(name="head", d=32, n_heads=2, head_dim=16, n_layers=2, ffn=64, window=3,
                n_groups=1, alpha=1.0, batch=2, seq_len=9, dtype="fp32", sigma=0.2)
    base.update(kw)
    return RLTConfig(**base)


def torch_encode(p, h, cfg, tokens):
    """The encoder written with torch library routines (causal SDPA) in float64."""
    t = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in p.items()}
    th = {k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in h.items()}
    x = th["embed"][torch.from_numpy(np.asarray(tokens, np.int64))]
    B, n, d = x.shape
    H, hd = cfg.n_heads, cfg.head_dim

    def heads(y):
        return y.view(B, n, H, hd).transpose(1, 2)

    for l in range(cfg.n_layers):
        a = F.rms_norm(x, (d,), th["enc_gamma"][l, 0], cfg.eps)
        q, k, v = (heads(a @ t[w][l]) for w in ("wq", "wk", "wv"))
        att = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        x = x + att.transpose(1, 2).reshape(B, n, d) @ t["wo"][l]
        f = F.rms_norm(x, (d,), th["enc_gamma"][l, 1], cfg.eps)
        x = x + (F.silu(f @ t["w1"][l]) * (f @ t["w3"][l])) @ t["w2"][l]
    return F.rms_norm(x, (d,), th["enc_gamma_out"], cfg.eps).numpy()


@pytest.fixture(scope="module")
def small():
    cfg = cfg_small()
    p = make_params(cfg, seed=1, random_gains=True)
    h = make_head_params(cfg, vocab=40, seed=1, random_gains=True)
    tok = make_tokens(range(cfg.batch), cfg.seq_len, vocab=40, seed=1)
    return cfg, p, h, tok


def test_encoder_matches_torch_causal_attention(small):
    cfg, p, h, tok = small
    got = oracle.encode(p, h, cfg, tok)
    ref = torch_encode(p, h, cfg, tok)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_encoder_is_causal(small):
    cfg, p, h, tok = small
    e = oracle.encode(p, h, cfg, tok)
    for t in (0, 3, cfg.seq_len - 2):
        tok2 = tok.copy()
        tok2[:, t + 1:] = (tok2[:, t + 1:] + 7) % 40
        e2 = oracle.encode(p, h, cfg, tok2)
        assert np.array_equal(e2[:, :t + 1], e[:, :t + 1])
        assert not np.array_equal(e2[:, t + 1:], e[:, t + 1:])


def test_encoder_uses_the_decoder_blocks_attention_and_ffn_matrices(small):
    cfg, p, h, tok = small
    e = oracle.encode(p, h, cfg, tok)
    p2 = dict(p)
    for name in ("wcq", "wco", "wmk", "wmv", "w_gate"):  # decoder-only weights
        p2[name] = p[name] * -3.0
    assert np.array_equal(oracle.encode(p2, h, cfg, tok), e)
    for name in ("wq", "wk", "wv", "wo", "w1", "w3", "w2"):  # shared with the encoder
        p3 = dict(p)
        p3[name] = p[name] * 1.5
        assert not np.allclose(oracle.encode(p3, h, cfg, tok), e)


def test_encoder_first_position_and_uniform_attention_closed_forms(small):
    cfg, p, h, tok = small
    # one position: attention over a single key returns its value
    x = np.asarray(h["embed"], np.float64)[tok[:, :1]]
    for l in range(cfg.n_layers):
        a = oracle.rms_norm(x, h["enc_gamma"][l, 0], cfg.eps)
        x = x + (a @ p["wv"][l]) @ p["wo"][l]
        f = oracle.rms_norm(x, h["enc_gamma"][l, 1], cfg.eps)
        x = x + (oracle.silu(f @ p["w1"][l]) * (f @ p["w3"][l])) @ p["w2"][l]
    e1 = oracle.rms_norm(x, h["enc_gamma_out"], cfg.eps)
    assert np.max(np.abs(oracle.encode(p, h, cfg, tok[:, :1]) - e1)) < 1e-12
    # zero query weights: every softmax is uniform, so position t averages values 1..t
    rng = np.random.default_rng(0)
    q = np.zeros((2, 5, 8))
    k, v = rng.standard_normal((2, 5, 8)), rng.standard_normal((2, 5, 8))
    out = oracle.causal_self_attention(q, k, v, 2)
    means = np.cumsum(v, axis=1) / np.arange(1, 6)[None, :, None]
    assert np.max(np.abs(out - means)) < 1e-12


def test_readout_matches_library_routines(small):
    cfg, p, h, tok = small
    s = np.random.default_rng(2).standard_normal((3, cfg.d))
    got = oracle.readout_logits(h, cfg, s)
    ref = (F.rms_norm(torch.from_numpy(s), (cfg.d,), torch.from_numpy(
        h["out_gamma"].astype(np.float64)), cfg.eps) @ torch.from_numpy(
        h["w_out"].astype(np.float64))).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12
    z = np.random.default_rng(3).standard_normal((4, 50)) * 5
    assert np.max(np.abs(oracle.log_softmax(z) - torch.log_softmax(torch.from_numpy(z), -1)
                         .numpy())) < 1e-12


def test_sampler_hand_worked_cases():
    with open(GOLDEN) as f:
        g = json.load(f)
    logits = np.log(np.array(g["probabilities"]))
    ev = {"log": math.log, "sqrt": math.sqrt}
    for c in g["cases"]:
        a, lb, lm, _ = oracle.sample(logits, c["temperature"], c["top_k"], c["top_p"], c["u"])
        assert a == c["token"], c
        assert abs(lb - eval(c["logp_behaviour"], {}, ev)) < 1e-12, c
        assert abs(lm - eval(c["logp_model"], {}, ev)) < 1e-12, c


def test_sampler_draws_exactly_the_truncated_distribution():
    """On a grid of N uniforms the inverse-CDF draw takes token a about N pi(a) times (within
    one draw); pi is the kept tokens' renormalised q, and the behaviour log-probabilities are
    log pi."""
    rng = np.random.default_rng(5)
    for temp, k, top_p in ((1.0, 0, 1.0), (0.7, 20, 1.0), (1.3, 0, 0.6), (1.0, 10, 0.9)):
        logits = rng.standard_normal(64) * 2
        N = 20000
        u = (np.arange(N) + 0.5) / N
        draws = [oracle.sample(logits, temp, k, top_p, x) for x in u]
        keep = draws[0][3]
        q = np.exp(logits / temp - np.max(logits / temp))
        q /= q.sum()
        pi = np.where(keep, q, 0) / q[keep].sum()
        counts = np.bincount([d[0] for d in draws], minlength=64)
        assert np.all(np.abs(counts - N * pi) <= 1.0 + 1e-9)
        assert not np.any(counts[~keep])
        for a, lb, _, _ in draws[:: N // 50]:
            assert abs(lb - np.log(pi[a])) < 1e-12
        # the kept tokens are the most probable ones
        if keep.sum() < 64:
            assert q[keep].min() >= q[~keep].max()
        if k:
            assert keep.sum() <= k


def test_sampler_limits_and_ties():
    rng = np.random.default_rng(6)
    z = rng.standard_normal(30)
    amax = int(np.argmax(z))
    for u in (0.0, 0.5, 0.999):
        a, lb, lm, _ = oracle.sample(z, 0.0, 0, 1.0, u)  # greedy
        assert a == amax and lb == 0.0
        a, lb, _, keep = oracle.sample(z, 1.0, 1, 1.0, u)  # top-1
        assert a == amax and abs(lb) < 1e-15 and keep.sum() == 1
        a, lb, _, keep = oracle.sample(z, 1.0, 0, 1e-9, u)  # smallest nucleus
        assert a == amax and keep.sum() == 1
    # untruncated at temperature 1: behaviour = model log-probability
    a, lb, lm, keep = oracle.sample(z, 1.0, 0, 1.0, 0.42)
    assert keep.all() and abs(lb - lm) < 1e-12
    assert abs(lm - oracle.log_softmax(z)[a]) < 1e-15
    # a shift of every logit changes nothing
    for args in ((0.8, 7, 0.9, 0.3), (1.0, 0, 0.5, 0.77)):
        r1 = oracle.sample(z, *args)
        r2 = oracle.sample(z + 123.0, *args)
        assert r1[0] == r2[0] and abs(r1[1] - r2[1]) < 1e-9 and np.array_equal(r1[3], r2[3])
    # ties: equal logits keep the lowest token ids first
    _, _, _, keep = oracle.sample(np.zeros(8), 1.0, 3, 1.0, 0.5)
    assert np.array_equal(np.flatnonzero(keep), [0, 1, 2])
    _, _, _, keep = oracle.sample(np.zeros(8), 1.0, 0, 0.3, 0.5)
    assert np.array_equal(np.flatnonzero(keep), [0, 1, 2])  # 3/8 >= 0.3 > 2/8
    # exact boundaries (every sum below is exact in binary): a prefix whose mass equals the
    # top-p target completes the nucleus, and a running sum equal to u does not exceed it
    _, _, _, keep = oracle.sample(np.zeros(8), 1.0, 0, 0.25, 0.5)
    assert np.array_equal(np.flatnonzero(keep), [0, 1])
    assert oracle.sample(np.zeros(4), 1.0, 0, 1.0, 0.5)[0] == 2
    assert oracle.sample(np.zeros(4), 1.0, 0, 1.0, 0.0)[0] == 0
    # greedy ties: the first maximal logit
    assert oracle.sample(np.array([0.0, 2.0, 2.0]), 0.0, 0, 1.0, 0.1)[0] == 1
