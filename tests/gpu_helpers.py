"""Shared helpers of the GPU tests: run the HIP path through the C-ABI binding and compare
with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import stateful_decoding_amd as sd
from synth import RLTConfig, make_encoder_outputs, make_params

TOL = {"fp32": 1e-4, "bf16": 3e-2}  # max relative L2 error of every s_t and every cache block


def max_rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    """max over leading indices of ||got - ref||_2 / ||ref||_2 along the last axis."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(num / np.maximum(den, 1e-30)))


def block_rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    """Caches [L, B, n, d]: relative L2 over each (layer, sequence) block, max over blocks."""
    g = np.asarray(got, np.float64).reshape(got.shape[0], got.shape[1], -1)
    r = np.asarray(ref, np.float64).reshape(ref.shape[0], ref.shape[1], -1)
    return max_rel_l2(g, r)


class GpuRun:
    """Model + state + memory for one configuration, driven through the C-ABI."""

    def __init__(self, cfg: RLTConfig, params: dict, batch: int, capacity: int, version: int = 7):
        self.cfg = cfg
        self.model = sd.Model(cfg, sd.upload_weights(params, sd.make_config(cfg)), version=version)
        self.state = sd.State(self.model, batch)
        self.mem = sd.Memory(self.model, batch, capacity)
        self.batch = batch

    def to_dev(self, e: np.ndarray) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(e)).to("cuda", self.model.dtype).contiguous()

    def run(self, e: np.ndarray) -> np.ndarray:
        """rlt_run_sequence over e [B, n, d]; returns s_traj [B, n, d] on the host."""
        ed = self.to_dev(e)
        traj = torch.empty(e.shape[0], e.shape[1], self.cfg.d, dtype=torch.float32, device="cuda")
        sd.rlt_run_sequence(self.model, self.state, self.mem, ed, traj)
        torch.cuda.synchronize()
        return traj.cpu().numpy()

    def export(self):
        s, k, v, n_valid, pos, ver = sd.rlt_state_export(self.state)
        return (s.cpu().numpy(), k.float().cpu().numpy(), v.float().cpu().numpy(), n_valid, pos,
                ver)


def oracle_run(cfg: RLTConfig, params: dict, e: np.ndarray):
    traj, st = oracle.run_sequence(params, cfg, e)
    K, V, n_valid = oracle.export_caches(cfg, st)
    return traj, K, V, n_valid


def check_against_oracle(cfg: RLTConfig, params: dict, e: np.ndarray, gpu_traj: np.ndarray,
                         gpu_snap, seqs=None, tol=None):
    """Compare GPU trajectories / final caches of sequences `seqs` with the oracle run on
    exactly those sequences. Returns (traj_err, k_err, v_err)."""
    seqs = list(range(e.shape[0])) if seqs is None else list(seqs)
    tol = TOL[cfg.dtype] if tol is None else tol
    traj, K, V, n_valid = oracle_run(cfg, params, e[seqs])
    err = max_rel_l2(gpu_traj[seqs], traj)
    s, k, v, nv, pos, _ = gpu_snap
    assert pos == e.shape[1] and nv == n_valid
    assert np.array_equal(s[seqs], gpu_traj[seqs, -1])
    ke = ve = 0.0
    if n_valid:
        ke = block_rel_l2(k[:, seqs, :n_valid], K[:, :, :n_valid])
        ve = block_rel_l2(v[:, seqs, :n_valid], V[:, :, :n_valid])
        assert not np.any(k[:, :, n_valid:]) and not np.any(v[:, :, n_valid:])
    assert err <= tol and ke <= tol and ve <= tol, (err, ke, ve, tol)
    return err, ke, ve


def inputs(cfg: RLTConfig, batch: int, seq_len: int, seed: int = 0, **kw):
    p = make_params(cfg, seed=seed, **kw)
    e = make_encoder_outputs(cfg, range(batch), seq_len=seq_len, seed=seed)
    return p, e


def export_host(g: GpuRun, seqs):
    """Snapshot of sequences `seqs` on the host in float64: (s, k, v, n_valid, position)."""
    s, k, v, n_valid, pos, _ = sd.rlt_state_export(g.state)
    idx = torch.tensor(list(seqs), device=s.device)
    out = (s.index_select(0, idx).double().cpu().numpy(),
           k.index_select(1, idx).double().cpu().numpy(),
           v.index_select(1, idx).double().cpu().numpy(), n_valid, pos)
    del s, k, v
    return out


def oracle_state_from_export(snap) -> oracle.OracleState:
    s, k, v, n_valid, pos = snap
    L = k.shape[0]
    return oracle.OracleState(
        s=s.copy(), cache_k=[[k[l, :, i] for i in range(n_valid)] for l in range(L)],
        cache_v=[[v[l, :, i] for i in range(n_valid)] for l in range(L)], t=pos)


def transition_parity(cfg: RLTConfig, params: dict, e: np.ndarray, sample_ts, seqs, tol=None):
    """Per-transition parity at 1-based tokens `sample_ts`.

    The GPU runs the whole sequence (rlt_run_sequence in chunks split around each sampled
    token); for every sampled t the oracle takes the GPU's exported state H_{t-1} of the
    sampled sequences, performs one transition with e_t, and its s_t and retained caches are
    compared with the GPU's H_t. Rounding differences therefore cannot compound through a
    recurrence that amplifies perturbations. Returns (GPU trajectory [B, T, d], max errors).
    """
    tol = TOL[cfg.dtype] if tol is None else tol
    B, T = e.shape[:2]
    seqs = list(seqs)
    g = GpuRun(cfg, params, B, T)
    pre, post, chunks, pos = {}, {}, [], 0
    for t in sorted(set(sample_ts)):
        if t - 1 > pos:
            chunks.append(g.run(e[:, pos:t - 1]))
            pos = t - 1
        pre[t] = export_host(g, seqs)
        chunks.append(g.run(e[:, pos:t]))
        pos = t
        post[t] = export_host(g, seqs)
    if pos < T:
        chunks.append(g.run(e[:, pos:]))
    traj = np.concatenate(chunks, axis=1)
    del g
    p = oracle.prepare_params(params)
    es = e[seqs].astype(np.float64)
    km, vm = oracle.memory_projection(p, es)
    worst = [0.0, 0.0, 0.0]
    for t in sorted(pre):
        st = oracle_state_from_export(pre[t])
        s_ref = oracle.decoder_step(p, cfg, st, km, vm, es[:, t - 1])
        K, V, nv = oracle.export_caches(cfg, st)
        s_gpu, k_gpu, v_gpu, nv_gpu, pos_gpu = post[t]
        assert (nv_gpu, pos_gpu) == (nv, t)
        errs = [max_rel_l2(s_gpu, s_ref)]
        if nv:
            # whole retained blocks, and the entry this transition appended on its own
            errs += [max(block_rel_l2(k_gpu[:, :, :nv], K[:, :, :nv]),
                         max_rel_l2(k_gpu[:, :, nv - 1], K[:, :, nv - 1])),
                     max(block_rel_l2(v_gpu[:, :, :nv], V[:, :, :nv]),
                         max_rel_l2(v_gpu[:, :, nv - 1], V[:, :, nv - 1]))]
        print(f"  transition t={t}: max rel L2 (s, k, v) = "
              + ", ".join(f"{x:.2e}" for x in errs), flush=True)
        assert max(errs) <= tol, (t, errs, tol)
        worst = [max(a, b) for a, b in zip(worst, errs + [0.0] * (3 - len(errs)))]
    return traj, worst
