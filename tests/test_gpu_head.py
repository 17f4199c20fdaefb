"""The encoder (rlt_encode) and the readout/sampler (rlt_readout) on the GPU against the oracle.

Encoder outputs and logits are compared row by row (relative L2 of every [d] row of e and every
[V] row of logits; 3e-2 for bf16, 1e-4 for fp32). The sampler's decisions are integers taken from
floating point: the oracle decides from the GPU's own logits (float64), and every action must
equal the oracle's, except where u (or the top-p target) lies within 1e-6 of a boundary of the
oracle's cumulative distribution; there the GPU's action must be one of the two tokens at that
boundary. Log-probabilities are compared within 1e-4 (they are computed in fp32 on the GPU).
"""
import numpy as np
import pytest
import torch

import oracle
import stateful_decoding_amd as sd
from synth import (CONFIGS, RLTConfig, make_head_params, make_params, make_tokens, make_uniforms,
                   round_bf16)
from tests.gpu_helpers import TOL, max_rel_l2

pytestmark = pytest.mark.gpu

MARGIN = 1e-6


def cfg_small(**kw):
    base = dict(name="head", d=128, n_heads=2, head_dim=64, n_layers=2, ffn=256, window=5,
                n_groups=1, alpha=1.0, batch=3, seq_len=24, dtype="bf16", sigma=0.05)
    base.update(kw)
    return RLTConfig(**base)


def setup(cfg, vocab, seed=0, head_sigma=None, dup_cols=(), tweak=None):
    p = make_params(cfg, seed=seed, random_gains=True, random_gate_bias=True)
    h = make_head_params(cfg, vocab=vocab, seed=seed, random_gains=True)
    if head_sigma is not None:
        h["w_out"] = (h["w_out"] * (head_sigma / cfg.sigma)).astype(np.float32)
    if tweak is not None:
        tweak(h)
    if cfg.dtype == "bf16":
        h["w_out"] = round_bf16(h["w_out"])
    for a, b in dup_cols:  # identical readout columns give bitwise identical logits
        h["w_out"][:, b] = h["w_out"][:, a]
    c = sd.make_config(cfg)
    model = sd.Model(c, sd.upload_weights(p, c))
    head = sd.Head(model, vocab, sd.upload_head_weights(h, c))
    return p, h, model, head


@pytest.mark.parametrize("case", [
    dict(head_dim=64, B=3, n=70),
    dict(head_dim=32, n_heads=4, B=2, n=33, n_layers=1),
    dict(head_dim=128, n_heads=2, d=256, ffn=512, B=2, n=130),
    dict(head_dim=64, B=5, n=1),
])
def test_encoder_matches_oracle(case):
    case = dict(case)
    B, n = case.pop("B"), case.pop("n")
    cfg = cfg_small(**case)
    p, h, model, head = setup(cfg, 512, seed=B + n)
    tok = make_tokens(range(B), n, vocab=512, seed=n)
    tok[0, 0] = 511  # the last id of the table
    e = sd.rlt_encode(head, torch.from_numpy(tok).cuda())
    torch.cuda.synchronize()
    ref = oracle.encode(p, h, cfg, tok)
    err = max_rel_l2(e.float().cpu().numpy(), ref)
    print(f"encoder d={cfg.d} hd={cfg.head_dim} L={cfg.n_layers} B={B} n={n}: max rel L2 "
          f"{err:.2e}", flush=True)
    assert err <= TOL["bf16"]


def test_encoder_full_size_sampled_and_feeds_the_decoder():
    """The 140M-scale workload's shapes (B = 256, n = 1024, V = 32768): every sequence is
    encoded in one launch sequence; sequence 0 (all 1024 positions) and sequence 255 (its first
    128) are checked against the oracle, and the encoder's output drives rlt_run_sequence."""
    cfg = CONFIGS["s140m_bf16"]
    B, n, V = cfg.batch, cfg.seq_len, 32768
    p, h, model, head = setup(cfg, V)
    tok = make_tokens(range(B), n, vocab=V)
    td = torch.from_numpy(tok).cuda()
    e = sd.rlt_encode(head, td)
    torch.cuda.synchronize()
    for b, m in ((0, n), (B - 1, 128)):
        ref = oracle.encode(p, h, cfg, tok[b:b + 1, :m])
        err = max_rel_l2(e[b:b + 1, :m].float().cpu().numpy(), ref)
        print(f"  sequence {b}, positions 1..{m}: max rel L2 {err:.2e}", flush=True)
        assert err <= TOL["bf16"]
    # the encoder's output is a valid decoder input
    state, mem = sd.State(model, B), sd.Memory(model, B, n)
    traj = torch.empty(B, 8, cfg.d, device="cuda")
    sd.rlt_run_sequence(model, state, mem, e[:, :8].contiguous(), traj)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(traj).all())


def check_samples(logits, temperature, top_k, top_p, u, tok, lpb, lpm):
    """Oracle decisions from the GPU's logits; returns the number of boundary cases."""
    near = 0
    for b in range(logits.shape[0]):
        z = logits[b].astype(np.float64)
        a, lb, lm, keep = oracle.sample(z, temperature, top_k, top_p, float(u[b]))
        g = int(tok[b])
        assert abs(lpm[b] - oracle.log_softmax(z)[g]) < 1e-4, b
        if g == a:
            assert abs(lpb[b] - lb) < 1e-4, (b, lpb[b], lb)
            continue
        # a different action is allowed only at a boundary of the oracle's distribution
        assert temperature > 0.0, (b, g, a)
        q = np.exp(z / temperature - np.max(z / temperature))
        q /= q.sum()
        idx = np.flatnonzero(keep)
        cdf = np.cumsum(q[idx]) / q[idx].sum()
        pos = int(np.searchsorted(idx, a))
        neighbours = {int(idx[j]) for j in (pos - 1, pos + 1) if 0 <= j < len(idx)}
        at_u = float(np.min(np.abs(cdf - u[b]))) < MARGIN and g in neighbours
        order = np.argsort(-z, kind="stable")
        top = order[: (len(z) if top_k <= 0 or top_k >= len(z) else top_k)]
        run = np.cumsum(q[top])
        at_p = top_p < 1.0 and float(np.min(np.abs(run - top_p * q[top].sum()))) < MARGIN
        assert at_u or at_p, (b, g, a, float(u[b]))
        near += 1
    return near


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_readout_logits_and_samples_match_oracle(dtype):
    cfg = cfg_small(dtype=dtype, d=128)
    B, V = 37, 4096
    p, h, model, head = setup(cfg, V, seed=3, head_sigma=0.2, dup_cols=((5, 9), (5, 700)))
    s = np.random.default_rng(4).standard_normal((B, cfg.d)).astype(np.float32) * 3
    sd_ = torch.from_numpy(s).cuda()
    ref = oracle.readout_logits(h, cfg, s)
    total_near = 0
    for i, (temp, k, tp) in enumerate(((1.0, 0, 1.0), (0.7, 0, 0.9), (1.5, 50, 1.0),
                                       (1.0, 10, 0.5), (0.0, 0, 1.0), (1.0, 1, 1.0),
                                       (2.0, V - 1, 0.3), (1.0, 2, 1.0))):
        u = make_uniforms(B, step=i)
        lg = torch.empty(B, V, device="cuda")
        tok, lpb, lpm = sd.rlt_readout(head, sd_, torch.from_numpy(u).cuda(), temp, k, tp,
                                       logits=lg)
        torch.cuda.synchronize()
        logits = lg.cpu().numpy()
        if i == 0:
            err = max_rel_l2(logits, ref)
            print(f"readout {dtype}: logits max rel L2 {err:.2e}", flush=True)
            assert err <= TOL[dtype]
            assert np.array_equal(logits[:, 5], logits[:, 9])
        tok, lpb, lpm = tok.cpu().numpy(), lpb.cpu().numpy(), lpm.cpu().numpy()
        if temp == 0.0:
            assert np.array_equal(tok, np.argmax(logits, axis=1)) and not np.any(lpb)
        near = check_samples(logits, temp, k, tp, u, tok, lpb, lpm)
        total_near += near
        print(f"  temperature {temp} top_k {k} top_p {tp}: {near} boundary cases", flush=True)
    assert total_near <= 2


def test_readout_large_vocabulary():
    """A vocabulary above the 32768 logits the sampler stages in LDS: every pass then reads
    the row from global memory. Same decisions as the oracle on the GPU's logits."""
    cfg = cfg_small()
    B, V = 6, 65536
    p, h, model, head = setup(cfg, V, seed=11, head_sigma=0.2, dup_cols=((7, 40000),))
    s = torch.from_numpy(np.random.default_rng(12).standard_normal((B, cfg.d)).astype(np.float32)
                         * 3).cuda()
    lg = torch.empty(B, V, device="cuda")
    near = 0
    for i, (temp, k, tp) in enumerate(((1.0, 0, 1.0), (0.8, 50, 0.95), (1.2, 0, 0.7),
                                       (0.0, 0, 1.0), (1.0, 40001, 1.0))):
        u = make_uniforms(B, step=20 + i)
        tok, lpb, lpm = sd.rlt_readout(head, s, torch.from_numpy(u).cuda(), temp, k, tp,
                                       logits=lg)
        torch.cuda.synchronize()
        near += check_samples(lg.cpu().numpy(), temp, k, tp, u, tok.cpu().numpy(),
                              lpb.cpu().numpy(), lpm.cpu().numpy())
    assert near <= 1


def test_sampler_ties_keep_the_lowest_ids():
    """Identical readout columns give identical logits; with top-k cutting through the tie
    group, only its lowest ids survive, so only they are ever sampled."""
    cfg = cfg_small()
    V = 1024
    B = 64
    s = np.tile(np.random.default_rng(6).standard_normal((1, cfg.d)).astype(np.float32), (B, 1))

    def tweak(h):  # column 3 along the normalised s: the largest logit by far
        a = oracle.rms_norm(s[0].astype(np.float64), h["out_gamma"], cfg.eps)
        h["w_out"][:, 3] = (a / np.linalg.norm(a) * 0.5).astype(np.float32)

    dup = tuple((3, j) for j in (17, 200, 512, 1000))
    p, h, model, head = setup(cfg, V, seed=5, head_sigma=0.05, dup_cols=dup, tweak=tweak)
    lg = torch.empty(B, V, device="cuda")
    u = (np.arange(B, dtype=np.float32) + 0.5) / B
    tok, lpb, lpm = sd.rlt_readout(head, torch.from_numpy(s).cuda(), torch.from_numpy(u).cuda(),
                                   1.0, 1, 1.0, logits=lg)
    torch.cuda.synchronize()
    z = lg[0].cpu().numpy()
    assert z[3] == z.max() and all(z[j] == z[3] for _, j in dup)
    # top-1 with a 5-way tie at the maximum: token 3 every time, probability 1
    assert np.all(tok.cpu().numpy() == 3) and np.all(np.abs(lpb.cpu().numpy()) < 1e-6)
    logits = lg.cpu().numpy()
    for k in (2, 3, 6):
        tok, lpb, lpm = sd.rlt_readout(head, torch.from_numpy(s).cuda(),
                                       torch.from_numpy(u).cuda(), 1.0, k, 1.0)
        torch.cuda.synchronize()
        assert check_samples(logits, 1.0, k, 1.0, u, tok.cpu().numpy(), lpb.cpu().numpy(),
                             lpm.cpu().numpy()) <= 1


def test_readout_is_deterministic_and_rejects_bad_arguments():
    cfg = cfg_small()
    V, B = 2048, 300
    p, h, model, head = setup(cfg, V, seed=7, head_sigma=0.1)
    s = torch.randn(B, cfg.d, device="cuda", generator=torch.Generator("cuda").manual_seed(1))
    u = torch.rand(B, device="cuda", generator=torch.Generator("cuda").manual_seed(2))
    a = sd.rlt_readout(head, s, u, 0.8, 100, 0.95)
    b = sd.rlt_readout(head, s, u, 0.8, 100, 0.95)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for bad in (dict(temperature=-1.0), dict(top_k=-2), dict(top_p=0.0), dict(top_p=1.5)):
        args = dict(temperature=1.0, top_k=0, top_p=1.0)
        args.update(bad)
        with pytest.raises(sd.RLTError) as ex:
            sd.rlt_readout(head, s, u, **args)
        assert ex.value.status_name == "RLT_ERR_ARG", bad
    with pytest.raises(sd.RLTError) as ex:
        sd.Head(model, 1000, sd.upload_head_weights(h, model.cfg))
    assert ex.value.status_name == "RLT_ERR_SHAPE"
    fp = cfg_small(dtype="fp32")
    p2, h2, m2, head2 = setup(fp, 512, seed=8)
    with pytest.raises(sd.RLTError):
        sd.rlt_encode(head2, torch.zeros(1, 4, dtype=torch.int32, device="cuda"))


def test_prompt_to_token_matches_oracle():
    """Tokens -> encoder -> memory + decoder run -> readout -> sample, end to end, against the
    oracle's own chain (bf16, small, contracting weights)."""
    cfg = cfg_small(sigma=0.05)
    B, n, V = 4, 20, 1024
    p, h, model, head = setup(cfg, V, seed=9, head_sigma=0.3)
    tok = make_tokens(range(B), n, vocab=V, seed=9)
    e = sd.rlt_encode(head, torch.from_numpy(tok).cuda())
    state, mem = sd.State(model, B), sd.Memory(model, B, n)
    traj = torch.empty(B, n, cfg.d, device="cuda")
    sd.rlt_run_sequence(model, state, mem, e, traj)
    u = make_uniforms(B, step=99)
    lg = torch.empty(B, V, device="cuda")
    t_gpu, lpb, lpm = sd.rlt_readout(head, traj[:, -1].contiguous(), torch.from_numpy(u).cuda(),
                                     0.9, 40, 0.95, logits=lg)
    torch.cuda.synchronize()
    e_ref = oracle.encode(p, h, cfg, tok)
    s_ref, _ = oracle.run_sequence(p, cfg, e_ref)
    lg_ref = oracle.readout_logits(h, cfg, s_ref[:, -1])
    errs = (max_rel_l2(e.float().cpu().numpy(), e_ref), max_rel_l2(traj.cpu().numpy(), s_ref),
            max_rel_l2(lg.cpu().numpy(), lg_ref))
    print(f"prompt to token: max rel L2 e {errs[0]:.2e}, s {errs[1]:.2e}, logits {errs[2]:.2e}",
          flush=True)
    assert max(errs) <= TOL["bf16"]
    assert check_samples(lg.cpu().numpy(), 0.9, 40, 0.95, u, t_gpu.cpu().numpy(),
                         lpb.cpu().numpy(), lpm.cpu().numpy()) <= 1
