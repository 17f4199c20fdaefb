"""Backpropagation through time on the GPU (rlt_bptt) against the float64 oracle's reverse
traversal (oracle.bptt), for the loss sum_{b,t} G[b, t] . s_t(b) with seeded random G.

Every gradient tensor is compared as a whole and row by row. The whole tensor's relative L2
error ||gpu - oracle|| / ||oracle|| is bounded by the figure of the forward parity (TOL: 1e-4
fp32, 3e-2 bf16). Every row along the last axis of each weight gradient (one input feature's
gradient over all outputs, per layer or group) and every [d] row of dLoss/de (one sequence and
token) also has its own relative L2 error, bounded by ROW_TOL, so a wrong layer, head, row or
token cannot hide inside the norm of a whole tensor: such a mistake leaves an error of the size
of the row itself.

ROW_TOL for bf16 is the whole-tensor bound times 10/3: the squared whole-tensor error is the
mean of the squared row errors (rows of similar size), and the largest of R roughly Gaussian
row errors exceeds their RMS by about sqrt(2 ln R), 3.0 to 4.8 for the 10^2 to 10^5 rows of
these tensors. fp32 rows keep 1e-4: their errors sit at 1e-7 to 1e-6. The denominator of a row
is its own norm, but never less than a quarter of its tensor's RMS row norm: a gradient row is
a sum of products over batch and tokens whose rounding error scales with the magnitudes of its
terms, i.e. with a typical row of the tensor, not with this row's (possibly cancelling) sum."""
import numpy as np
import pytest
import torch

import oracle
import stateful_decoding_amd as sd
from synth import CONFIGS, RLTConfig
from tests.gpu_helpers import TOL, inputs, max_rel_l2

pytestmark = pytest.mark.gpu


def cfg_small(**kw):
    base = dict(name="bptt", d=64, n_heads=2, head_dim=32, n_layers=2, ffn=128, window=3,
                n_groups=2, alpha=0.7, batch=3, seq_len=10, dtype="fp32", sigma=0.05)
    base.update(kw)
    return RLTConfig(**base)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


ROW_TOL = {"fp32": 1e-4, "bf16": 1e-1}  # largest per-row error (module docstring)
ROW_FLOOR = 0.25  # a row's denominator is at least this fraction of its tensor's RMS row norm


def row_rel_l2(got, ref, zero_scale: float):
    """(whole-tensor, largest per-row) relative L2 error of one gradient tensor, rows along
    the last axis.

    A tensor whose exact gradient is zero (every row of the query and key weights when the
    window holds one token) is judged on `zero_scale`, the typical row norm of the loss's
    other gradients, so a rounding residue passes and a real leak does not. Rows are judged on
    at least ROW_FLOOR times their tensor's RMS row norm (the module docstring says why)."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    g = g.reshape(-1, g.shape[-1]) if g.ndim > 1 else g.reshape(1, -1)
    r = r.reshape(-1, r.shape[-1]) if r.ndim > 1 else r.reshape(1, -1)
    num = np.linalg.norm(g - r, axis=-1)
    den = np.linalg.norm(r, axis=-1)
    rms = float(np.sqrt(np.mean(den ** 2)))
    if rms == 0:
        x = float(np.linalg.norm(g) / zero_scale)
        return x, float(np.max(num) / zero_scale)
    whole = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    return whole, float(np.max(num / np.maximum(den, ROW_FLOOR * rms)))


def grad_errors(got: dict, ref: dict) -> dict:
    """(whole-tensor, largest per-row) relative L2 error of every gradient tensor
    (row_rel_l2). The scale for exactly-zero tensors is the mean RMS row norm of the nonzero
    gradient tensors."""
    rms = []
    for k in oracle.GRAD_NAMES:
        r = np.asarray(ref[k], np.float64)
        r = r.reshape(-1, r.shape[-1]) if r.ndim > 1 else r.reshape(1, -1)
        x = float(np.sqrt(np.mean(np.sum(r * r, axis=-1))))
        if x > 0:
            rms.append(x)
    scale = float(np.mean(rms))
    return {k: row_rel_l2(got[k], ref[k], scale) for k in oracle.GRAD_NAMES}


def de_errors(got, ref):
    """(whole, largest per-row) relative L2 error of dLoss/de, rows of one sequence and token."""
    r = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    den = np.linalg.norm(r, axis=-1)
    scale = float(np.sqrt(np.mean(den[den > 0] ** 2))) if np.any(den > 0) else 1.0
    return row_rel_l2(got, ref, scale)


def check(errs: dict, dtype: str):
    """Every (whole, row) pair within (TOL, ROW_TOL); plain floats (s_traj) within TOL."""
    print("  rel L2 (whole/row):", " ".join(
        f"{k}={v[0]:.1e}/{v[1]:.1e}" if isinstance(v, tuple) else f"{k}={v:.1e}"
        for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        whole, row = v if isinstance(v, tuple) else (v, 0.0)
        assert whole <= TOL[dtype] and row <= ROW_TOL[dtype], (k, whole, row)


def run_case(cfg, B, T, seed):
    p, e = inputs(cfg, B, T, seed=seed, random_gains=True, random_gate_bias=True)
    G = np.random.default_rng(seed + 1000).standard_normal((B, T, cfg.d)).astype(np.float32)
    model = sd.Model(cfg, sd.upload_weights(p, sd.make_config(cfg)))
    ed = torch.from_numpy(np.ascontiguousarray(e)).to("cuda", model.dtype).contiguous()
    Gd = torch.from_numpy(G).cuda()
    grads = sd.grad_buffers(model)
    de = torch.empty(B, T, cfg.d, dtype=torch.float32, device="cuda")
    traj = torch.empty(B, T, cfg.d, dtype=torch.float32, device="cuda")
    print(f"case d={cfg.d} hd={cfg.head_dim} L={cfg.n_layers} F={cfg.ffn} W={cfg.window} "
          f"G={cfg.n_groups} alpha={cfg.alpha} {cfg.dtype} B={B} T={T}", flush=True)
    sd.rlt_bptt(model, ed, Gd, grads, de=de, s_traj=traj)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in grads.items()}
    ref_traj, ref, ref_de = oracle.bptt(p, cfg, e, G)
    errs = grad_errors(got, ref)
    errs["de"] = de_errors(de.cpu().numpy(), ref_de)
    errs["s_traj"] = max_rel_l2(traj.cpu().numpy(), ref_traj)
    return errs


CASES = [
    dict(dtype="fp32", B=3, T=10),                                               # G = L
    dict(dtype="fp32", B=2, T=9, n_groups=1, alpha=1.0, window=4, head_dim=64, n_heads=1),
    dict(dtype="fp32", B=4, T=7, window=1, n_layers=1, n_groups=1),             # W = 1
    dict(dtype="bf16", B=5, T=24, d=128, n_heads=2, head_dim=64, ffn=256, window=5),
    dict(dtype="bf16", B=3, T=12, d=256, n_heads=2, head_dim=128, ffn=512, window=20,
         n_groups=1),                                                            # W > T
    dict(dtype="bf16", B=300, T=40, d=128, n_heads=4, head_dim=32, ffn=192, window=6),
    dict(dtype="fp32", B=2, T=6, d=256, n_heads=2, head_dim=128, ffn=256, window=2),
    dict(dtype="bf16", B=3, T=1, d=128, n_heads=2, head_dim=64, ffn=256, window=5),  # one token
    # d and F multiples of 128 in bf16: the weight gradients of all layers are formed by one
    # batched launch per weight kind on the gradient stream. 272 sequences make 16-token
    # chunks, so 40 tokens take three chunks, using both copies of the chunk buffers, with
    # loss on every token
    dict(dtype="bf16", B=272, T=40, d=128, n_heads=2, head_dim=64, ffn=256, window=6),
]


@pytest.mark.parametrize("case", CASES)
def test_bptt_matches_oracle(case):
    case = dict(case)
    B, T = case.pop("B"), case.pop("T")
    cfg = cfg_small(**case)
    check(run_case(cfg, B, T, seed=B + T), cfg.dtype)


def test_bptt_chunked_rows_span_several_weight_gradient_chunks():
    """B = 300 sequences make 14-token weight-gradient chunks, so 40 tokens take three
    chunks, the first one short; fp32 holds that bookkeeping to the tight bound."""
    cfg = cfg_small(dtype="fp32", d=64, ffn=128, window=5)
    check(run_case(cfg, 300, 40, seed=3), "fp32")


def test_bptt_argument_errors():
    cfg = cfg_small()
    p, e = inputs(cfg, 2, 4)
    model = sd.Model(cfg, sd.upload_weights(p, sd.make_config(cfg)))
    ed = torch.from_numpy(np.ascontiguousarray(e)).to("cuda", model.dtype).contiguous()
    Gd = torch.zeros(2, 4, cfg.d, device="cuda")
    grads = sd.grad_buffers(model)
    ws = sd.bptt_workspace(model, 2, 4)
    with pytest.raises(sd.RLTError) as ex:
        sd.rlt_bptt(model, ed, Gd, grads, ws=ws[: ws.numel() // 2])
    assert ex.value.status_name == "RLT_ERR_CAPACITY"
    lib = model.lib
    g = sd.binding.rlt_grads(*[grads[k].data_ptr() for k in sd.binding.WEIGHT_FIELDS])
    g.w2 = None
    st = lib.rlt_bptt(model.handle, ed.data_ptr(), 2, 4, Gd.data_ptr(), None,
                      sd.binding.byref(g), None, ws.data_ptr(), ws.numel(), None, None, None,
                      None)
    assert sd.binding.STATUS_NAMES[st] == "RLT_ERR_ARG"
    g.w2 = grads["w2"].data_ptr()
    for seg, bits in ((0, 1), (2, 4)):
        tr = sd.binding.rlt_truncation(seg, bits)
        st = lib.rlt_bptt(model.handle, ed.data_ptr(), 2, 4, Gd.data_ptr(), None,
                          sd.binding.byref(g), None, ws.data_ptr(), ws.numel(),
                          sd.binding.byref(tr), None, None, None)
        assert sd.binding.STATUS_NAMES[st] == "RLT_ERR_ARG", (seg, bits)


def test_full_size_bptt_early_tokens_match_oracle():
    """The benchmark's launch configuration (the 140M-scale workload, B = 256, T = 1024): the
    whole forward and the whole reverse walk run, with the loss restricted to sequences 0 and
    255 at tokens 1..16. Every gradient then equals the oracle's for those two sequences over
    those 16 tokens, and dLoss/de is exactly zero for every other sequence and later token."""
    cfg = CONFIGS["s140m_bf16"]
    B, T, n_or = cfg.batch, cfg.seq_len, 16
    seqs = [0, B - 1]
    p, e = inputs(cfg, B, T)
    G = np.zeros((B, T, cfg.d), np.float32)
    G[seqs, :n_or] = np.random.default_rng(7).standard_normal((2, n_or, cfg.d))
    model = sd.Model(cfg, sd.upload_weights(p, sd.make_config(cfg)))
    ed = torch.from_numpy(e).to("cuda", model.dtype).contiguous()
    Gd = torch.from_numpy(G).cuda()
    del e
    grads = sd.grad_buffers(model)
    de = torch.empty(B, T, cfg.d, dtype=torch.float32, device="cuda")
    print(f"full size {cfg.name}: B={B} T={T}, loss on sequences {seqs} tokens 1..{n_or}",
          flush=True)
    sd.rlt_bptt(model, ed, Gd, grads, de=de)
    torch.cuda.synchronize()
    e_or = ed[seqs, :n_or].float().cpu().numpy()
    _, ref, ref_de = oracle.bptt(p, cfg, e_or, G[seqs, :n_or])
    errs = grad_errors({k: v.cpu().numpy() for k, v in grads.items()}, ref)
    de_h = de.cpu().numpy()
    errs["de"] = de_errors(de_h[seqs, :n_or], ref_de)
    mask = np.ones(B, bool)
    mask[seqs] = False
    assert not np.any(de_h[mask]) and not np.any(de_h[seqs, n_or:])
    check(errs, "bf16")


@pytest.mark.parametrize("B", [5, 300])
def test_bptt_forward_equals_decoder_path(B):
    """The forward inside rlt_bptt runs the decoder-step kernels with the same row groups as
    rlt_run_sequence, writing its saves on the side, except that it keeps the output projection
    and the cross-attention query as the two products it differentiates, where the decoder step
    computes them in one fused launch (a reassociation): the trajectories agree within the
    forward's bound."""
    cfg = cfg_small(dtype="bf16", d=128, n_heads=2, head_dim=64, ffn=256, window=4)
    T = 12
    p, e = inputs(cfg, B, T, seed=B)
    model = sd.Model(cfg, sd.upload_weights(p, sd.make_config(cfg)))
    ed = torch.from_numpy(np.ascontiguousarray(e)).to("cuda", model.dtype).contiguous()
    traj = torch.empty(B, T, cfg.d, dtype=torch.float32, device="cuda")
    sd.rlt_bptt(model, ed, torch.zeros(B, T, cfg.d, device="cuda"), sd.grad_buffers(model),
                s_traj=traj)
    state, mem = sd.State(model, B), sd.Memory(model, B, T)
    ref = torch.empty_like(traj)
    sd.rlt_run_sequence(model, state, mem, ed, ref)
    torch.cuda.synchronize()
    err = max_rel_l2(traj.cpu().numpy(), ref.cpu().numpy())
    print(f"  training forward vs decoder path: max rel L2 {err:.2e}", flush=True)
    assert err <= TOL["bf16"]


def test_bptt_feedback_zero_start_state_gradient_is_exactly_zero():
    """With alpha = 0 nothing flows back into s_{t-1}: the start state's gradient is exactly
    zero and the rest still matches the oracle."""
    cfg = cfg_small(dtype="bf16", d=128, n_heads=2, head_dim=64, ffn=256, window=5, alpha=0.0)
    check(run_case(cfg, 4, 20, seed=11), "bf16")
    p, e = inputs(cfg, 4, 20, seed=11, random_gains=True, random_gate_bias=True)
    model = sd.Model(cfg, sd.upload_weights(p, sd.make_config(cfg)))
    ed = torch.from_numpy(np.ascontiguousarray(e)).to("cuda", model.dtype).contiguous()
    grads = sd.grad_buffers(model)
    sd.rlt_bptt(model, ed, torch.randn(4, 20, cfg.d, device="cuda"), grads)
    torch.cuda.synchronize()
    assert not torch.any(grads["s_star"])


def test_bptt_is_deterministic_across_calls():
    """No atomics and fixed reduction orders: two calls (two row groups on two streams) give
    bitwise identical gradients."""
    cfg = cfg_small(dtype="bf16", d=128, n_heads=2, head_dim=64, ffn=256, window=6)
    B, T = 272, 20
    p, e = inputs(cfg, B, T, seed=21)
    model = sd.Model(cfg, sd.upload_weights(p, sd.make_config(cfg)))
    ed = torch.from_numpy(np.ascontiguousarray(e)).to("cuda", model.dtype).contiguous()
    ds = torch.randn(B, T, cfg.d, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    ws = sd.bptt_workspace(model, B, T)
    runs = []
    for _ in range(2):
        g = sd.grad_buffers(model)
        de = torch.empty(B, T, cfg.d, device="cuda")
        sd.rlt_bptt(model, ed, ds, g, de=de, ws=ws)
        torch.cuda.synchronize()
        runs.append((g, de))
    for k in sd.binding.WEIGHT_FIELDS:
        assert torch.equal(runs[0][0][k], runs[1][0][k]), k
    assert torch.equal(runs[0][1], runs[1][1])


TRUNC_CASES = [
    dict(dtype="fp32", B=3, T=13, segment=4, detach=("state", "window"), window=3),
    dict(dtype="fp32", B=2, T=11, segment=3, detach=("state",), window=5, n_groups=1),
    dict(dtype="fp32", B=2, T=10, segment=4, detach=("window",), window=6),
    dict(dtype="bf16", B=5, T=24, segment=5, detach=("state", "window"), d=128, n_heads=2,
         head_dim=64, ffn=256, window=7),
    dict(dtype="bf16", B=300, T=30, segment=8, detach=("state", "window"), d=128, n_heads=4,
         head_dim=32, ffn=192, window=6),
    dict(dtype="fp32", B=2, T=9, segment=1, detach=("state", "window"), window=4),
    dict(dtype="fp32", B=2, T=9, segment=20, detach=("state", "window"), window=4),
]


@pytest.mark.parametrize("case", TRUNC_CASES)
def test_truncated_bptt_matches_oracle(case):
    """Truncated backpropagation (segment length k, named detached tensors) against the
    oracle's truncated reverse traversal; segment 1 cuts at every token, a segment longer than
    the sequence cuts nothing."""
    case = dict(case)
    B, T = case.pop("B"), case.pop("T")
    seg, det = case.pop("segment"), case.pop("detach")
    cfg = cfg_small(**case)
    p, e = inputs(cfg, B, T, seed=B + T + seg, random_gains=True, random_gate_bias=True)
    G = np.random.default_rng(seg).standard_normal((B, T, cfg.d)).astype(np.float32)
    model = sd.Model(cfg, sd.upload_weights(p, sd.make_config(cfg)))
    ed = torch.from_numpy(np.ascontiguousarray(e)).to("cuda", model.dtype).contiguous()
    grads = sd.grad_buffers(model)
    de = torch.empty(B, T, cfg.d, dtype=torch.float32, device="cuda")
    print(f"truncated case {cfg.dtype} B={B} T={T} W={cfg.window} segment={seg} "
          f"detach={det}", flush=True)
    sd.rlt_bptt(model, ed, torch.from_numpy(G).cuda(), grads, de=de, segment=seg, detach=det)
    torch.cuda.synchronize()
    _, ref, ref_de = oracle.bptt(p, cfg, e, G, segment=seg, detach=det)
    errs = grad_errors({k: v.cpu().numpy() for k, v in grads.items()}, ref)
    errs["de"] = de_errors(de.cpu().numpy(), ref_de)
    check(errs, cfg.dtype)


def test_detaching_the_state_alone_leaves_the_window_path_open():
    """With the memory projections zeroed and the loss on the second segment only, detaching
    the state alone still sends gradient into the first segment's encoder outputs (through the
    window's keys and values); detaching the window too leaves exactly zero there."""
    cfg = cfg_small(dtype="fp32", window=4, n_groups=1)
    B, T, k = 2, 8, 4
    p, e = inputs(cfg, B, T, seed=5, random_gains=True, random_gate_bias=True)
    p = dict(p)
    p["wmk"] = np.zeros_like(p["wmk"])
    p["wmv"] = np.zeros_like(p["wmv"])
    G = np.zeros((B, T, cfg.d), np.float32)
    G[:, k:] = np.random.default_rng(1).standard_normal((B, T - k, cfg.d))
    model = sd.Model(cfg, sd.upload_weights(p, sd.make_config(cfg)))
    ed = torch.from_numpy(np.ascontiguousarray(e)).to("cuda", model.dtype).contiguous()
    out = {}
    for det in (("state",), ("state", "window")):
        de = torch.empty(B, T, cfg.d, dtype=torch.float32, device="cuda")
        sd.rlt_bptt(model, ed, torch.from_numpy(G).cuda(), sd.grad_buffers(model), de=de,
                    segment=k, detach=det)
        torch.cuda.synchronize()
        out[det] = de.cpu().numpy()
        _, _, ref_de = oracle.bptt(p, cfg, e, G, segment=k, detach=det)
        assert rel_l2(out[det], ref_de) <= TOL["fp32"], det
    leak = np.linalg.norm(out[("state",)][:, :k], axis=-1)
    assert np.all(leak > 0)
    assert not np.any(out[("state", "window")][:, :k])


def test_bptt_clock_timing_leaves_gradients_unchanged():
    """The backward attention kernels timed by their own clock stamps (every launch of both
    row groups) give the same gradients bitwise as an untimed pass; a clock buffer too small
    for the pass is reported after it."""
    cfg = cfg_small(dtype="bf16", d=128, n_heads=2, head_dim=64, ffn=256, window=4)
    B, T = 272, 10
    p, e = inputs(cfg, B, T, seed=4)
    model = sd.Model(cfg, sd.upload_weights(p, sd.make_config(cfg)))
    ed = torch.from_numpy(np.ascontiguousarray(e)).to("cuda", model.dtype).contiguous()
    ds = torch.randn(B, T, cfg.d, device="cuda", generator=torch.Generator("cuda").manual_seed(5))
    ws = sd.bptt_workspace(model, B, T)
    ref = sd.grad_buffers(model)
    sd.rlt_bptt(model, ed, ds, ref, ws=ws)
    slots = T * cfg.n_layers * B * cfg.n_heads  # one per workgroup of each launch of one kind
    got = sd.grad_buffers(model)
    stats = sd.rlt_bptt(model, ed, ds, got, ws=ws, time_kernels=["bwd_cross_attn",
                                                                 "bwd_self_attn"],
                        clock=sd.clock_buffer(2 * slots))
    torch.cuda.synchronize()
    for k in sd.binding.WEIGHT_FIELDS:
        assert torch.equal(got[k], ref[k]), k
    groups = 2  # 272 sequences: two row groups
    for k in ("bwd_cross_attn", "bwd_self_attn"):
        assert stats[k]["launches"] == T * cfg.n_layers * groups, k
        assert 0 < stats[k]["total_ms"] < 1e3, k
    with pytest.raises(sd.RLTError) as ex:
        sd.rlt_bptt(model, ed, ds, got, ws=ws, time_kernels=["bwd_cross_attn", "bwd_self_attn"],
                    clock=sd.clock_buffer(slots))
    assert ex.value.status_name == "RLT_ERR_CAPACITY"
