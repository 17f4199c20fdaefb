"""Ragged ready updates (rlt_decoder_step_ragged): sequences of one batch advance only when
active, each at its own position; the result for every sequence must be exactly its own
token-by-token recurrence, as the oracle computes it for that sequence alone."""
import numpy as np
import pytest
import torch

import stateful_decoding_amd as sd
from synth import RLTConfig
from tests.gpu_helpers import TOL, GpuRun, block_rel_l2, inputs, max_rel_l2, oracle_run

pytestmark = pytest.mark.gpu


def cfg_small(**kw):
    base = dict(name="ragged", d=128, n_heads=2, head_dim=64, n_layers=2, ffn=256, window=4,
                n_groups=2, alpha=1.0, batch=5, seq_len=24, dtype="bf16", sigma=0.05)
    base.update(kw)
    return RLTConfig(**base)


def step(g, e_rows, active, B, d):
    s = torch.empty(B, d, dtype=torch.float32, device="cuda")
    act = None if active is None else torch.from_numpy(active.astype(np.uint8)).cuda()
    sd.rlt_decoder_step_ragged(g.model, g.state, g.mem, g.to_dev(e_rows), act, s)
    return s.cpu().numpy()


@pytest.mark.parametrize("case", [
    dict(B=5, steps=24, dtype="bf16"),
    dict(B=37, steps=20, dtype="fp32", window=3, head_dim=32, n_heads=4),
    dict(B=300, steps=12, dtype="bf16", window=6),  # two row groups on two streams
    # 12 sequence-head pairs and prefixes past 511 entries: the memory attention is split in
    # two slices per row, merged by a second launch; the rarely ready row leaves its second
    # slice empty
    dict(B=3, steps=700, dtype="fp32", window=5, head_dim=32, n_heads=4, n_layers=1,
         n_groups=1, probs=(0.9, 0.6, 0.01)),
])
def test_ragged_schedule_matches_oracle(case):
    case = dict(case)
    B, steps = case.pop("B"), case.pop("steps")
    probs = np.array(case.pop("probs", (0.6,) * B))
    cfg = cfg_small(**case)
    T = steps
    p, e = inputs(cfg, B, T, seed=B + steps, random_gains=True, random_gate_bias=True)
    g = GpuRun(cfg, p, B, T)
    sd.rlt_memproj(g.model, g.mem, g.to_dev(e), 0)  # memory of every token is known up front
    rng = np.random.default_rng(B * 31 + steps)
    pos = np.zeros(B, dtype=np.int64)
    outs = {b: [] for b in range(B)}
    s_prev = np.broadcast_to(p["s_star"].astype(np.float32), (B, cfg.d)).copy()
    for i in range(steps):
        active = rng.random(B) < probs
        if i == 3:
            active[:] = False  # a step where nothing is ready
        rows = np.stack([e[b, min(pos[b], T - 1)] for b in range(B)])
        s = step(g, rows, active, B, cfg.d)
        for b in range(B):
            if active[b]:
                outs[b].append(s[b])
                pos[b] += 1
            else:
                # inactive rows report their unchanged s
                assert np.array_equal(s[b], s_prev[b]), (i, b)
        s_prev = s
    torch.cuda.synchronize()
    assert g.state.positions() == pos.tolist()
    assert g.state.position == -1
    snap_s, snap_k, snap_v, nv, position, _ = g.export()
    assert nv == -1 and position == -1
    worst = 0.0
    for b in range(B):
        n = int(pos[b])
        if n == 0:
            assert np.array_equal(snap_s[b], p["s_star"].astype(np.float32))
            continue
        traj, K, V, n_valid = oracle_run(cfg, p, e[b:b + 1, :n])
        worst = max(worst, max_rel_l2(np.stack(outs[b])[None], traj))
        assert np.array_equal(snap_s[b], outs[b][-1])
        if n_valid:
            worst = max(worst, block_rel_l2(snap_k[:, b:b + 1, :n_valid], K[:, :, :n_valid]),
                        block_rel_l2(snap_v[:, b:b + 1, :n_valid], V[:, :, :n_valid]))
        assert not np.any(snap_k[:, b, n_valid:]) and not np.any(snap_v[:, b, n_valid:])
    print(f"  ragged B={B}: max rel L2 over every active s_t and cache block: {worst:.3e}",
          flush=True)
    assert worst <= TOL[cfg.dtype]


def test_all_active_ragged_step_equals_uniform_step():
    cfg = cfg_small()
    B, T = 7, 9
    p, e = inputs(cfg, B, T, seed=4)
    a = GpuRun(cfg, p, B, T)
    full = a.run(e)
    b = GpuRun(cfg, p, B, T)
    sd.rlt_memproj(b.model, b.mem, b.to_dev(e), 0)
    got = []
    for i in range(T):
        active = np.ones(B, bool) if i % 2 else None  # explicit mask or NULL
        got.append(step(b, e[:, i], active, B, cfg.d))
    assert np.array_equal(np.stack(got, 1), full)
    assert b.state.positions() == [T] * B


def test_ragged_step_needs_projected_memory():
    cfg = cfg_small()
    B, T = 3, 6
    p, e = inputs(cfg, B, T, seed=2)
    g = GpuRun(cfg, p, B, T)
    sd.rlt_memproj(g.model, g.mem, g.to_dev(e[:, :2]), 0)
    act = np.array([1, 0, 1], bool)
    step(g, e[:, 0], act, B, cfg.d)
    step(g, e[:, 1], act, B, cfg.d)
    with pytest.raises(sd.RLTError) as ex:  # a sequence may be at position 2: entry 3 is missing
        step(g, e[:, 2], act, B, cfg.d)
    assert ex.value.status_name == "RLT_ERR_NOT_PROJECTED"
    with pytest.raises(sd.RLTError) as ex:  # positions differ: run_sequence cannot project
        sd.rlt_run_sequence(g.model, g.state, g.mem, g.to_dev(e[:, 2:4]))
    assert ex.value.status_name == "RLT_ERR_NOT_PROJECTED"
    assert g.state.positions() == [2, 0, 2]


def test_ragged_snapshot_split_and_resume():
    """Export a batch whose sequences are at different positions, import it into a fresh
    state, and continue both with the same ragged steps: bitwise the same."""
    cfg = cfg_small(window=5)
    B, T = 6, 16
    p, e = inputs(cfg, B, T, seed=9)
    a = GpuRun(cfg, p, B, T)
    sd.rlt_memproj(a.model, a.mem, a.to_dev(e), 0)
    rng = np.random.default_rng(3)
    pos = np.zeros(B, dtype=np.int64)
    masks = [rng.random(B) < 0.6 for _ in range(12)]
    for m in masks[:7]:
        step(a, np.stack([e[b, min(pos[b], T - 1)] for b in range(B)]), m, B, cfg.d)
        pos += m
    assert a.state.positions() == pos.tolist()
    s, k, v, _, _, ver = sd.rlt_state_export(a.state)
    b = GpuRun(cfg, p, B, T)
    sd.rlt_memproj(b.model, b.mem, b.to_dev(e), 0)
    sd.rlt_state_import_ragged(b.state, s, k, v, pos.tolist(), ver)
    assert b.state.positions() == pos.tolist()
    for m in masks[7:]:
        rows = np.stack([e[i, min(pos[i], T - 1)] for i in range(B)])
        out_a = step(a, rows, m, B, cfg.d)
        out_b = step(b, rows, m, B, cfg.d)
        assert np.array_equal(out_a, out_b)
        pos += m
    sa, sb = sd.rlt_state_export(a.state), sd.rlt_state_export(b.state)
    for x, y in zip(sa[:3], sb[:3]):
        assert torch.equal(x, y)
