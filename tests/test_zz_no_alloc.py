"""rlt_run_parallel_noalloc (the token-parallel pass with the library's own scratch array as
workspace) against rlt_run_parallel with a caller workspace: two calls in a row on one GPU, the
second with a smaller input, each equal to the workspace path bitwise (same kernels, same
operands), and a pass too large for the array refused before any work."""
import numpy as np
import pytest
import torch

import stateful_decoding_amd as sd
from synth import RLTConfig
from tests.gpu_helpers import GpuRun, inputs

pytestmark = pytest.mark.gpu


def cfg_a0(**kw):
    base = dict(name="noalloc_a0", d=128, n_heads=2, head_dim=64, n_layers=2, ffn=256,
                window=5, n_groups=2, alpha=0.0, batch=3, seq_len=24, dtype="bf16",
                sigma=0.05)
    base.update(kw)
    return RLTConfig(**base)


def one_pass(cfg, B, T, seed, noalloc):
    p, e = inputs(cfg, B, T, seed=seed, random_gains=True, random_gate_bias=True)
    g = GpuRun(cfg, p, B, T)
    ed = g.to_dev(e)
    traj = torch.empty(B, T, cfg.d, dtype=torch.float32, device="cuda")
    if noalloc:
        sd.rlt_run_parallel_noalloc(g.model, g.state, g.mem, ed, traj)
    else:
        sd.rlt_run_parallel(g.model, g.state, g.mem, ed, traj)
    torch.cuda.synchronize()
    return traj.cpu().numpy(), g.export()


def test_noalloc_equals_workspace_path_on_two_calls():
    cfg = cfg_a0()
    lib = sd.load_library()
    assert lib.rlt_scratch_bytes() == 64 << 20
    for B, T, seed in ((6, 150, 1), (3, 70, 2)):  # the second call is smaller
        assert lib.rlt_parallel_ws_bytes(sd.make_config(cfg), B, T) <= lib.rlt_scratch_bytes()
        print(f"noalloc pass B={B} T={T}", flush=True)
        ref, ref_snap = one_pass(cfg, B, T, seed, noalloc=False)
        got, snap = one_pass(cfg, B, T, seed, noalloc=True)
        assert np.array_equal(got, ref)
        for x, y in zip(snap[:3], ref_snap[:3]):
            assert np.array_equal(x, y)
        assert snap[3:] == ref_snap[3:]


def test_noalloc_refuses_a_pass_beyond_the_scratch_array():
    cfg = cfg_a0(d=512, n_heads=8, head_dim=64, ffn=2048, n_layers=1, n_groups=1)
    lib = sd.load_library()
    B, T = 4, 2048  # about 80 MB of workspace
    assert lib.rlt_parallel_ws_bytes(sd.make_config(cfg), B, T) > lib.rlt_scratch_bytes()
    p, e = inputs(cfg, B, 1, seed=3)
    g = GpuRun(cfg, p, B, T)
    ed = torch.zeros(B, T, cfg.d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sd.RLTError) as ex:
        sd.rlt_run_parallel_noalloc(g.model, g.state, g.mem, ed)
    assert ex.value.status_name == "RLT_ERR_CAPACITY"
    assert g.state.position == 0 and g.mem.length == 0
