"""Parity of the HIP path (through the C-ABI) with the CPU oracle, on the GPU.

Small cases compare every s_t and the final caches of every sequence; they span several
GEMM tiles, ragged batch tails, windows of 1 and 2, shared and per-layer memory, the
feedback scale at 0 and negative, random gains, every head size and both dtypes, and memory
prefixes long enough to be split over several workgroups. Full-size workloads run in the
benchmark's launch configuration and are compared on sampled sequences.
"""
import numpy as np
import pytest
import torch

import stateful_decoding_amd as sd
from synth import CONFIGS, RLTConfig
import oracle
from tests.gpu_helpers import (TOL, GpuRun, check_against_oracle, inputs, max_rel_l2,
                               transition_parity)

pytestmark = pytest.mark.gpu


def cfg_small(**kw):
    base = dict(name="small", d=128, n_heads=2, head_dim=64, n_layers=2, ffn=256, window=5,
                n_groups=1, alpha=1.0, batch=3, seq_len=24, dtype="bf16", sigma=0.05)
    base.update(kw)
    return RLTConfig(**base)


def run_case(cfg, B, T, seed=0, seqs=None, **kw):
    p, e = inputs(cfg, B, T, seed=seed, **kw)
    print(f"case {cfg.name} d={cfg.d} hd={cfg.head_dim} L={cfg.n_layers} W={cfg.window} "
          f"G={cfg.n_groups} a={cfg.alpha} {cfg.dtype} B={B} T={T}", flush=True)
    g = GpuRun(cfg, p, B, T)
    traj = g.run(e)
    errs = check_against_oracle(cfg, p, e, traj, g.export(), seqs=seqs)
    print("  max rel L2 (s, k, v):", errs, flush=True)
    return g, p, e, traj


def test_tiny_fp32_config():
    cfg = CONFIGS["tiny_fp32"]
    run_case(cfg, cfg.batch, cfg.seq_len)


@pytest.mark.parametrize("case", [
    dict(dtype="fp32", head_dim=32, n_heads=4, window=4, B=37, T=20),
    dict(dtype="fp32", head_dim=64, window=1, B=5, T=12),
    dict(dtype="fp32", head_dim=128, n_heads=1, window=2, n_groups=2, B=17, T=15),
    dict(dtype="bf16", head_dim=32, n_heads=4, window=3, alpha=0.0, B=9, T=16),
    dict(dtype="bf16", head_dim=64, window=7, n_groups=2, alpha=-0.5, B=33, T=30),
    dict(dtype="bf16", head_dim=128, n_heads=2, d=256, ffn=512, window=9, B=5, T=70,
         sigma=0.03),
    dict(dtype="bf16", head_dim=64, window=16, B=3, T=300),
    # few sequence-head pairs and long prefixes: the memory attention splits every prefix into
    # up to 4 (fp32) or 5 (bf16) slices and merges them in a second launch
    dict(dtype="fp32", head_dim=32, n_heads=4, window=6, B=3, T=1100, n_layers=1),
    dict(dtype="bf16", head_dim=128, n_heads=2, d=256, ffn=512, window=9, B=2, T=1400,
         n_layers=1, sigma=0.03),
    dict(dtype="fp32", head_dim=64, window=33, B=2, T=200, n_layers=1),
    # batches of >= 256 sequences run as row groups on separate streams
    dict(dtype="bf16", head_dim=64, window=6, n_groups=2, B=300, T=40),
    dict(dtype="fp32", head_dim=32, n_heads=4, window=3, B=256, T=12),
])
def test_small_cases(case):
    case = dict(case)
    B, T = case.pop("B"), case.pop("T")
    cfg = cfg_small(**case)
    run_case(cfg, B, T, seed=B + T, random_gains=True, random_gate_bias=True)


def test_memory_projection_matches_oracle():
    cfg = cfg_small(n_groups=2, dtype="fp32")
    p, e = inputs(cfg, 7, 19, seed=3)
    g = GpuRun(cfg, p, 7, 40)
    sd.rlt_memproj(g.model, g.mem, g.to_dev(e[:, :11]), 0)
    sd.rlt_memproj(g.model, g.mem, g.to_dev(e[:, 11:]), 11)
    assert g.mem.length == 19
    K, V = (x.float().cpu().numpy() for x in g.mem.views())
    km, vm = oracle.memory_projection(oracle.prepare_params(p), e.astype(np.float64))
    H, hd = cfg.n_heads, cfg.head_dim
    for got, ref in ((K, km), (V, vm)):
        ref = ref.reshape(2, 7, 19, H, hd).transpose(0, 1, 3, 2, 4)
        assert max_rel_l2(got[:, :, :, :19], ref) < 1e-5


def test_memory_projection_bf16_large_ragged_rows():
    """A bf16 projection of 37 x 451 = 16,687 rows (not a multiple of the 128-row tiles) into
    N = 2 groups x 2d = 1024 columns: enough workgroups (264) for the 256 x 256 token GEMM. Each
    entry is a bf16 rounding of an fp32-accumulated product, so the relative L2 error against
    the float64 oracle is bounded by half a bf16 ulp (2^-9) plus accumulation error."""
    cfg = cfg_small(dtype="bf16", d=256, n_heads=4, head_dim=64, ffn=512, n_groups=2)
    B, T = 37, 451
    p, e = inputs(cfg, B, T, seed=8)
    g = GpuRun(cfg, p, B, T)
    sd.rlt_memproj(g.model, g.mem, g.to_dev(e), 0)
    K, V = (x.float().cpu().numpy() for x in g.mem.views())
    km, vm = oracle.memory_projection(oracle.prepare_params(p), e.astype(np.float64))
    H, hd = cfg.n_heads, cfg.head_dim
    for got, ref in ((K, km), (V, vm)):
        ref = ref.reshape(2, B, T, H, hd).transpose(0, 1, 3, 2, 4)
        assert max_rel_l2(got[:, :, :, :T], ref) < 2.5e-3


@pytest.mark.parametrize("B", [6, 280])
def test_decoder_steps_equal_run_sequence_and_split(B):
    cfg = cfg_small(window=4, n_groups=2)
    T = 17
    p, e = inputs(cfg, B, T, seed=11)
    a = GpuRun(cfg, p, B, T)
    full = a.run(e)
    # memproj + n decoder steps
    b = GpuRun(cfg, p, B, T)
    sd.rlt_memproj(b.model, b.mem, b.to_dev(e), 0)
    outs = []
    for i in range(T):
        s = torch.empty(B, cfg.d, dtype=torch.float32, device="cuda")
        sd.rlt_decoder_step(b.model, b.state, b.mem, b.to_dev(e[:, i]), s)
        outs.append(s.cpu().numpy())
    assert np.array_equal(np.stack(outs, 1), full)
    # chunked run_sequence (memory projected chunk by chunk) == one run (Proposition 3.1)
    c = GpuRun(cfg, p, B, T)
    parts = [c.run(e[:, :5]), c.run(e[:, 5:6]), c.run(e[:, 6:])]
    assert np.array_equal(np.concatenate(parts, 1), full)
    # a run over tokens whose memory is partly projected already
    d = GpuRun(cfg, p, B, T)
    sd.rlt_memproj(d.model, d.mem, d.to_dev(e[:, :9]), 0)
    assert np.array_equal(d.run(e), full)
    # two fresh runs are bitwise identical
    assert np.array_equal(GpuRun(cfg, p, B, T).run(e), full)


def test_snapshot_roundtrip_and_reset():
    cfg = cfg_small(window=6)
    B, T, t1 = 4, 20, 8
    p, e = inputs(cfg, B, T, seed=12)
    g = GpuRun(cfg, p, B, T, version=99)
    full = g.run(e)
    h = GpuRun(cfg, p, B, T, version=99)
    h.run(e[:, :t1])
    s, k, v, nv, pos, ver = sd.rlt_state_export(h.state)
    assert (nv, pos, ver) == (min(t1, cfg.window - 1), t1, 99)
    h.run(e[:, t1:])  # continue, then rewind to the snapshot
    sd.rlt_state_import(h.state, s, k, v, pos, ver)
    assert h.state.position == t1
    rest = torch.empty(B, T - t1, cfg.d, dtype=torch.float32, device="cuda")
    sd.rlt_run_sequence(h.model, h.state, h.mem, h.to_dev(e[:, t1:]), rest)
    assert np.array_equal(rest.cpu().numpy(), full[:, t1:])
    with pytest.raises(sd.RLTError) as ex:
        sd.rlt_state_import(h.state, s, k, v, pos, 98)
    assert ex.value.status_name == "RLT_ERR_VERSION"
    assert h.state.position == T
    # reset returns to s* and an empty cache
    h.model.lib.rlt_state_reset(h.state.handle, None)
    s0, k0, _, nv0, pos0, _ = sd.rlt_state_export(h.state)
    assert pos0 == 0 and nv0 == 0 and not k0.any()
    assert np.array_equal(s0.cpu().numpy(), np.broadcast_to(p["s_star"], (B, cfg.d)))


def test_errors_are_reported_before_any_work():
    cfg = cfg_small()
    p, e = inputs(cfg, 2, 4)
    g = GpuRun(cfg, p, 2, 4)
    with pytest.raises(sd.RLTError) as ex:  # no memory projected yet
        sd.rlt_decoder_step(g.model, g.state, g.mem, g.to_dev(e[:, 0]))
    assert ex.value.status_name == "RLT_ERR_NOT_PROJECTED"
    assert g.state.position == 0
    with pytest.raises(sd.RLTError) as ex:  # beyond the memory capacity
        sd.rlt_run_sequence(g.model, g.state, g.mem, g.to_dev(np.concatenate([e, e], 1)))
    assert ex.value.status_name == "RLT_ERR_CAPACITY"
    with pytest.raises(sd.RLTError) as ex:  # hole in the memory
        sd.rlt_memproj(g.model, g.mem, g.to_dev(e[:, :1]), 2)
    assert ex.value.status_name == "RLT_ERR_NOT_PROJECTED"
    other = sd.State(g.model, 3)
    with pytest.raises(sd.RLTError) as ex:  # batch mismatch
        sd.rlt_run_sequence(g.model, other, g.mem, torch.zeros(3, 1, cfg.d, dtype=torch.bfloat16,
                                                                 device="cuda"))
    assert ex.value.status_name == "RLT_ERR_SHAPE"
    with pytest.raises(sd.RLTError) as ex:  # timing stride must be positive
        g.state.profile_begin(["cross_attn"], token_stride=0)
    assert ex.value.status_name == "RLT_ERR_ARG"


def test_kernel_timing_counts_sampled_launches():
    """Timed launches: every kind in the steps of tokens t % stride == 0, bytes as stated."""
    cfg = cfg_small(n_layers=2, window=3)
    B, T = 5, 11
    p, e = inputs(cfg, B, T)
    g = GpuRun(cfg, p, B, T)
    g.state.profile_begin(token_stride=4)
    g.run(e)
    prof = g.state.profile_end()
    steps = len(range(0, T, 4))  # tokens 0, 4, 8
    assert prof["memproj"]["launches"] == 1
    assert prof["gate"]["launches"] == steps
    for k in ("qkv", "self_attn", "self_out", "cross_attn", "cross_out", "ffn_up", "ffn_down"):
        assert prof[k]["launches"] == steps * cfg.n_layers, k
        assert prof[k]["total_ms"] > 0
    # the cross-attention query is computed by the fused output projection ("self_out")
    assert prof.get("cross_q", {}).get("launches", 0) == 0
    es = 2 if cfg.dtype == "bf16" else 4
    # memory attention reads t entries of K and V per sequence and layer at token t (1-based)
    kv = sum(B * (t + 1) * 2 * cfg.d * es for t in range(0, T, 4)) * cfg.n_layers
    act = steps * cfg.n_layers * B * cfg.d * (4 + es)
    assert prof["cross_attn"]["bytes"] == pytest.approx(kv + act)


def test_kernel_clock_timing_leaves_results_unchanged():
    """With a clock buffer attached the attention kernels time themselves (every launch of
    every row group), the other kinds keep their events, the trajectories stay bitwise equal to
    an untimed run, and a buffer too small for the session is reported."""
    cfg = cfg_small(n_layers=2, window=3)
    B, T = 300, 9
    p, e = inputs(cfg, B, T)
    g = GpuRun(cfg, p, B, T)
    ref = g.run(e)
    groups = min(4, max(1, B // 128))  # row groups of at least 128 sequences
    n_attn = T * cfg.n_layers * groups
    slots = T * cfg.n_layers * B * cfg.n_heads  # one per workgroup of each launch of one kind
    g.state.profile_clock(2 * slots)
    g.state.reset()
    g.mem.reset()
    g.state.profile_begin(["qkv", "self_attn", "cross_attn"], token_stride=1)
    got = g.run(e)
    prof = g.state.profile_end()
    assert np.array_equal(got, ref)
    for k in ("qkv", "self_attn", "cross_attn"):
        assert prof[k]["launches"] == n_attn, k
        assert 0 < prof[k]["total_ms"] < 1e3, k
    g.state.profile_clock(slots)  # room for one attention kind but not for both
    g.state.reset()
    g.mem.reset()
    g.state.profile_begin(["self_attn", "cross_attn"], token_stride=1)
    g.run(e)
    with pytest.raises(sd.RLTError) as ex:
        g.state.profile_end()
    assert ex.value.status_name == "RLT_ERR_CAPACITY"
    g.state.profile_clock(None)
    g.state.reset()
    g.mem.reset()
    g.state.profile_begin(["cross_attn"], token_stride=1)
    g.run(e)
    assert g.state.profile_end()["cross_attn"]["launches"] == n_attn


# --- full-size workloads, sampled sequences ---------------------------------------------------
#
# With these random weights the recurrence of the ~140M-scale and long-context (alpha = 1)
# workloads amplifies perturbations: in the float64 oracle itself, a 1e-6 relative change
# of s* grows to ~1e-2 within 256 tokens (tests/test_oracle_dynamics.py). A trajectory from
# s* can then only be compared over its first tokens; every transition, however, can be
# compared exactly: the oracle steps from the GPU's own exported state.

def _full_size(name, T=None, seqs=(0,), sample_ts=(1,), traj_T=0):
    cfg = CONFIGS[name]
    T = cfg.seq_len if T is None else T
    B = cfg.batch
    print(f"full size {name}: B={B} T={T}, sequences {list(seqs)}, transitions at "
          f"{list(sample_ts)}, trajectory over {traj_T} tokens", flush=True)
    p, e = inputs(cfg, B, T)
    traj, worst = transition_parity(cfg, p, e, sample_ts, seqs)
    assert np.all(np.isfinite(traj))
    # the chunked runs above equal one rlt_run_sequence over all T tokens, bitwise (the
    # benchmark's launch configuration)
    g = GpuRun(cfg, p, B, T)
    assert np.array_equal(g.run(e), traj)
    del g
    if traj_T:
        ref, _ = oracle.run_sequence(p, cfg, e[list(seqs), :traj_T])
        err = max_rel_l2(traj[list(seqs), :traj_T], ref)
        per_t = [max_rel_l2(traj[list(seqs), t], ref[:, t]) for t in range(traj_T)]
        print(f"  trajectory from s*, first {traj_T} tokens: max rel L2 {err:.2e} (by token: "
              + " ".join(f"{x:.1e}" for x in per_t[::max(1, traj_T // 8)]) + ")", flush=True)
        assert err <= TOL[cfg.dtype]
    return p, e, traj


def test_full_size_s50m():
    # stable recurrence: the whole 1024-token trajectory is compared as well
    _full_size("s50m_bf16", seqs=(0, 37, 63), sample_ts=(1, 63, 64, 65, 1024), traj_T=1024)


@pytest.mark.timeout(900)
def test_full_size_s140m_bench_configuration():
    # the benchmark's workload: one rlt_run_sequence over B=256, T=1024 (two row groups of 128
    # sequences: rows 127 and 128 are the last of the first group and the first of the second).
    # The trajectory from s* is compared over 16 tokens: in the float64 oracle this recurrence
    # multiplies a relative perturbation of s* by 2.0 within 16 tokens, 2.6 within 32, 6.6
    # within 64 and over 1e3 within 256 (tests/test_oracle_dynamics.py), so a longer horizon
    # measures that amplification rather than the kernels; every sampled transition is compared
    # from the GPU's own state.
    _full_size("s140m_bf16", seqs=(0, 1, 64, 127, 128, 191, 254, 255),
               sample_ts=(1, 2, 127, 128, 129, 256, 384, 512, 640, 768, 896, 1024), traj_T=16)


@pytest.mark.timeout(1200)
def test_full_size_depth48():
    # the 48-layer workload at its stated length T = 4096: memory prefixes beyond 1024 entries
    # at head size 128, and the caches retained after the last token
    _full_size("depth48_bf16", seqs=(0, 31), sample_ts=(1, 255, 256, 257, 1024, 2048, 4096),
               traj_T=16)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["long_a1_bf16", "long_a0_bf16"])
def test_full_size_long_context(name):
    cfg = CONFIGS[name]
    p, e, traj = _full_size(name, seqs=(0, 15), sample_ts=(1, 128, 129, 4096, 8192),
                            traj_T=1024 if cfg.alpha == 0.0 else 32)
    if cfg.alpha == 0.0:
        # feedback off: a different start state changes nothing, bitwise, at full size
        p2 = dict(p)
        p2["s_star"] = p["s_star"][::-1].copy() * 3
        g2 = GpuRun(cfg, p2, e.shape[0], e.shape[1])
        assert np.array_equal(g2.run(e), traj)
