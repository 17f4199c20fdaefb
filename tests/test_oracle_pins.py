"""Pins of the CPU oracle against things other than itself (CPU only).

* a hand-worked whole step (tests/golden/hand_w1_l1_d2.json);
* an independent brute-force formulation (tests/brute_force.py);
* invariants the pages fix: window retention, prefix restriction of the memory, the
  feedback scale at zero, shared vs per-layer memory, the prompt/response split
  (Proposition 3.1), independence of sequences;
* library routines and closed forms for the sub-steps.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import RLTConfig, make_encoder_outputs, make_params, round_bf16
from tests.brute_force import brute_force_trajectory

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(**kw):
    base = dict(name="pin", d=16, n_heads=2, head_dim=8, n_layers=2, ffn=24, window=3,
                n_groups=1, alpha=1.0, batch=3, seq_len=8, dtype="fp32", sigma=0.3)
    base.update(kw)
    return RLTConfig(**base)


def tiny_inputs(cfg, seed=0):
    p = make_params(cfg, seed=seed, random_gains=True, random_gate_bias=True)
    e = make_encoder_outputs(cfg, range(cfg.batch), seed=seed)
    return p, e


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)))


# --- hand-worked case ---------------------------------------------------------------------

def _load_hand_case():
    with open(os.path.join(GOLDEN, "hand_w1_l1_d2.json")) as f:
        g = json.load(f)
    c = g["config"]
    cfg = RLTConfig("hand", c["d"], c["n_heads"], c["head_dim"], c["n_layers"], c["ffn"],
                    c["window"], c["n_groups"], c["alpha"], 1, 1, "fp32", 1.0, eps=c["eps"])
    p = {}
    for k, v in g["params"].items():
        p[k] = np.array([math.log(3.0) if x == "ln3" else x for x in v], np.float64) \
            if k == "b_gate" else np.array(v, np.float64)
    return g, cfg, p, np.array(g["e"], np.float64)


def test_hand_worked_step_closed_form():
    g, cfg, p, e = _load_hand_case()
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))  # noqa: E731
    closed = [7 + sig(1) - 7 * sig(-1), -1 - 14 * sig(-1)]
    np.testing.assert_allclose(closed, g["expected_s1"], rtol=0, atol=1e-14)
    traj, st = oracle.run_sequence(p, cfg, e)
    np.testing.assert_allclose(traj[0, 0], g["expected_s1"], rtol=0, atol=1e-12)
    K, V, n_valid = oracle.export_caches(cfg, st)
    assert n_valid == 0 and K.shape == (1, 1, 0, 2)


def test_hand_worked_cache_window_two():
    # At t = 1 a window of 2 still holds only the current token, so s_1 is unchanged and
    # the retained entry is this token's key/value.
    g, cfg, p, e = _load_hand_case()
    cfg = cfg.replace(window=2)
    traj, st = oracle.run_sequence(p, cfg, e)
    np.testing.assert_allclose(traj[0, 0], g["expected_s1"], rtol=0, atol=1e-12)
    K, V, n_valid = oracle.export_caches(cfg, st)
    assert n_valid == 1
    np.testing.assert_allclose(K[0, 0, 0], g["expected_cache_after_t1_with_window_2"]["k"],
                               atol=1e-12)
    np.testing.assert_allclose(V[0, 0, 0], g["expected_cache_after_t1_with_window_2"]["v"],
                               atol=1e-12)


# --- brute force ---------------------------------------------------------------------------

@pytest.mark.parametrize("window,groups,alpha", [
    (1, 1, 1.0), (2, 1, 1.0), (3, 2, 0.6), (4, 1, 0.0), (20, 2, 1.0), (3, 1, -0.8),
])
def test_oracle_matches_brute_force(window, groups, alpha):
    cfg = tiny(window=window, n_groups=groups, alpha=alpha)
    p, e = tiny_inputs(cfg, seed=window)
    traj, st = oracle.run_sequence(p, cfg, e)
    ref, hk, hv = brute_force_trajectory(p, cfg, e, return_history=True)
    assert rel_err(traj, ref) < 1e-12
    # retained caches are exactly the last W-1 keys/values of the full history
    K, V, n_valid = oracle.export_caches(cfg, st)
    T = cfg.seq_len
    assert n_valid == min(T, window - 1)
    if n_valid:
        np.testing.assert_allclose(K[:, :, :n_valid], hk[:, :, T - n_valid:], rtol=1e-12,
                                   atol=1e-12)
        np.testing.assert_allclose(V[:, :, :n_valid], hv[:, :, T - n_valid:], rtol=1e-12,
                                   atol=1e-12)


def test_brute_force_mask_ignores_entries_outside_window():
    cfg = tiny(window=2, seq_len=6)
    p, e = tiny_inputs(cfg, seed=3)
    a = brute_force_trajectory(p, cfg, e)
    b = brute_force_trajectory(p, cfg, e, perturb_outside_window=torch.Generator().manual_seed(1))
    assert np.array_equal(a, b)


def test_full_window_equals_causal_attention():
    # With W >= T the sliding window is plain causal self-attention: the result cannot
    # depend on W beyond that point.
    cfg = tiny(window=9, seq_len=8)
    p, e = tiny_inputs(cfg, seed=4)
    a, _ = oracle.run_sequence(p, cfg, e)
    b, _ = oracle.run_sequence(p, cfg.replace(window=50), e)
    assert np.array_equal(a, b)


# --- invariants ----------------------------------------------------------------------------

def test_prefix_restriction_of_memory():
    cfg = tiny(seq_len=8)
    p, e = tiny_inputs(cfg, seed=5)
    base, _ = oracle.run_sequence(p, cfg, e)
    for t in (1, 4, 7):
        e2 = e.copy()
        e2[:, t:] += np.random.default_rng(t).standard_normal(e2[:, t:].shape)
        pert, _ = oracle.run_sequence(p, cfg, e2)
        assert np.array_equal(base[:, :t], pert[:, :t])
        assert not np.allclose(base[:, t:], pert[:, t:])


def test_alpha_zero_removes_feedback():
    cfg = tiny(alpha=0.0)
    p, e = tiny_inputs(cfg, seed=6)
    a, _ = oracle.run_sequence(p, cfg, e)
    p2 = dict(p)
    p2["s_star"] = p["s_star"] + 5.0 * np.random.default_rng(0).standard_normal(cfg.d)
    b, _ = oracle.run_sequence(p2, cfg, e)
    assert np.array_equal(a, b)
    # a state injected mid-sequence has no influence either
    pp = oracle.prepare_params(p)
    km, vm = oracle.memory_projection(pp, e.astype(np.float64))
    st = oracle.init_state(pp, cfg, cfg.batch)
    for i in range(3):
        oracle.decoder_step(pp, cfg, st, km, vm, e[:, i].astype(np.float64))
    st.s = np.random.default_rng(1).standard_normal(st.s.shape) * 10
    c = oracle.decoder_step(pp, cfg, st, km, vm, e[:, 3].astype(np.float64))
    assert np.array_equal(c, a[:, 3])


def test_alpha_nonzero_feedback_matters():
    cfg = tiny(alpha=1.0)
    p, e = tiny_inputs(cfg, seed=6)
    a, _ = oracle.run_sequence(p, cfg, e)
    p2 = dict(p)
    p2["s_star"] = p["s_star"] + 1.0
    b, _ = oracle.run_sequence(p2, cfg, e)
    assert not np.allclose(a[:, 0], b[:, 0])


def test_shared_memory_equals_tied_layer_memories():
    cfg1 = tiny(n_groups=1)
    p, e = tiny_inputs(cfg1, seed=7)
    a, _ = oracle.run_sequence(p, cfg1, e)
    cfgL = cfg1.replace(n_groups=cfg1.n_layers)
    pL = dict(p)
    pL["wmk"] = np.repeat(p["wmk"], cfg1.n_layers, axis=0)
    pL["wmv"] = np.repeat(p["wmv"], cfg1.n_layers, axis=0)
    b, _ = oracle.run_sequence(pL, cfgL, e)
    assert np.array_equal(a, b)
    # untied layer memories do change the result
    pL["wmv"] = pL["wmv"].copy()
    pL["wmv"][1] *= -1
    c, _ = oracle.run_sequence(pL, cfgL, e)
    assert not np.allclose(a, c)


@pytest.mark.parametrize("split", [1, 3, 7])
def test_split_invariance(split):
    # Proposition 3.1 ("RLT Runs 96 Blocks Per Token...", section "Three design
    # principles"): where the prompt/response boundary falls does not change the state.
    cfg = tiny(seq_len=8, window=3)
    p, e = tiny_inputs(cfg, seed=8)
    pp = oracle.prepare_params(p)
    mem = oracle.memory_projection(pp, e.astype(np.float64))
    full, st_full = oracle.run_sequence(pp, cfg, e, memory=mem)
    a, st = oracle.run_sequence(pp, cfg, e[:, :split], memory=mem)
    b, st = oracle.run_sequence(pp, cfg, e[:, split:], state=st, memory=mem)
    assert np.array_equal(full, np.concatenate([a, b], axis=1))
    assert st.t == st_full.t == cfg.seq_len
    for l in range(cfg.n_layers):
        assert all(np.array_equal(x, y) for x, y in zip(st.cache_k[l], st_full.cache_k[l]))


def test_sequences_are_independent():
    cfg = tiny(batch=4)
    p, e = tiny_inputs(cfg, seed=9)
    a, _ = oracle.run_sequence(p, cfg, e)
    perm = [2, 0, 3, 1]
    b, _ = oracle.run_sequence(p, cfg, e[perm])
    assert rel_err(b, a[perm]) < 1e-13
    c, _ = oracle.run_sequence(p, cfg.replace(batch=1), e[1:2])
    assert rel_err(c, a[1:2]) < 1e-13


# --- sub-steps against library routines and closed forms ---------------------------------

@pytest.mark.parametrize("n,heads", [(1, 1), (5, 2), (17, 4), (40, 3)])
def test_attend_matches_library_sdpa(n, heads):
    rng = np.random.default_rng(n)
    B, hd = 3, 8
    d = heads * hd
    q, k, v = (rng.standard_normal(s) * 2 for s in ((B, d), (B, n, d), (B, n, d)))
    got = oracle.attend(q, k, v, heads)
    tq = torch.from_numpy(q).view(B, 1, heads, hd).transpose(1, 2)
    tk = torch.from_numpy(k).view(B, n, heads, hd).transpose(1, 2)
    tv = torch.from_numpy(v).view(B, n, heads, hd).transpose(1, 2)
    ref = F.scaled_dot_product_attention(tq, tk, tv).transpose(1, 2).reshape(B, d).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attend_closed_forms():
    rng = np.random.default_rng(0)
    B, n, d, H = 2, 6, 12, 3
    k, v = rng.standard_normal((B, n, d)), rng.standard_normal((B, n, d))
    # a zero query weighs all keys equally: the output is the mean of the values
    np.testing.assert_allclose(oracle.attend(np.zeros((B, d)), k, v, H), v.mean(axis=1),
                               rtol=1e-13, atol=1e-14)
    # a single key returns its value exactly
    q = rng.standard_normal((B, d)) * 100
    assert np.array_equal(oracle.attend(q, k[:, :1], v[:, :1], H), v[:, 0])
    # huge scores select the best-matching key (softmax limit)
    kk = np.zeros((B, n, d))
    kk[:, 2] = 1.0
    out = oracle.attend(np.full((B, d), 1e4), kk, v, H)
    np.testing.assert_allclose(out, v[:, 2], rtol=1e-12, atol=1e-12)


def test_rms_norm_silu_sigmoid_match_library():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 33)) * 3
    gam = rng.standard_normal(33)
    ref = F.rms_norm(torch.from_numpy(x), (33,), weight=torch.from_numpy(gam), eps=1e-6)
    np.testing.assert_allclose(oracle.rms_norm(x, gam, 1e-6), ref.numpy(), rtol=1e-13,
                               atol=1e-14)
    np.testing.assert_allclose(oracle.silu(x), F.silu(torch.from_numpy(x)).numpy(),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.sigmoid(x), torch.sigmoid(torch.from_numpy(x)).numpy(),
                               rtol=1e-13, atol=1e-15)
    assert oracle.sigmoid(np.array([-1000.0]))[0] == 0.0


def test_gate_merge_limits():
    # g -> 1 passes e_t through; g -> 0 passes alpha * s_{t-1} through.
    d = 4
    rng = np.random.default_rng(2)
    e, s = rng.standard_normal((2, d)), rng.standard_normal((2, d))
    p = {"w_gate": np.zeros((2 * d, d)), "b_gate": np.full(d, 800.0)}
    np.testing.assert_array_equal(oracle.gate_merge(p, 0.7, e, s), e)
    p["b_gate"] = np.full(d, -800.0)
    np.testing.assert_allclose(oracle.gate_merge(p, 0.7, e, s), 0.7 * s, rtol=0, atol=0)


def test_memory_projection_shapes_and_values():
    cfg = tiny(n_groups=2)
    p, e = tiny_inputs(cfg, seed=10)
    km, vm = oracle.memory_projection(oracle.prepare_params(p), e.astype(np.float64))
    assert km.shape == (2, cfg.batch, cfg.seq_len, cfg.d)
    np.testing.assert_allclose(
        vm[1, 2, 5], torch.from_numpy(e[2, 5].astype(np.float64)) @ torch.from_numpy(
            p["wmv"][1].astype(np.float64)), rtol=1e-13)


# --- input generator ------------------------------------------------------------------------

def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_bf16(x), ref)


def test_generator_streams_are_per_tensor_and_per_sequence():
    cfg = tiny(batch=4)
    e_all = make_encoder_outputs(cfg, range(4))
    e_two = make_encoder_outputs(cfg, [3, 1])
    assert np.array_equal(e_two, e_all[[3, 1]])
    e_short = make_encoder_outputs(cfg, [2], seq_len=3)
    assert np.array_equal(e_short[0], e_all[2, :3])
    p1 = make_params(cfg)
    p2 = make_params(cfg.replace(n_layers=3))
    assert np.array_equal(p1["wq"], p2["wq"][:2])
