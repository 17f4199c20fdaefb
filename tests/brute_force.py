"""Brute-force formulation of the RLT decoder recurrence, used only to pin the CPU oracle.

It shares no code with ``oracle/`` and is written differently on purpose:

* no ring buffer: every decoder key/value ever produced is kept, and each attention call
  selects what the token may see with an explicit boolean position mask, the window
  [t - W + 1, t] for self-attention and the prefix [1, t] for cross-attention (the
  architecture section of "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets");
* the encoder memory is projected once for the whole sequence and masked, never sliced;
* every s_t is recomputed from the learned start state s* (nothing carried between
  targets);
* the sub-steps are torch float64 library routines (scaled_dot_product_attention,
  rms_norm, silu, sigmoid) instead of hand-written NumPy.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _t(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64))


def _sdpa(q, keys, values, mask, n_heads):
    B, n, d = keys.shape
    hd = d // n_heads
    qh = q.reshape(B, 1, n_heads, hd).transpose(1, 2)
    kh = keys.reshape(B, n, n_heads, hd).transpose(1, 2)
    vh = values.reshape(B, n, n_heads, hd).transpose(1, 2)
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask.view(1, 1, 1, n))
    return o.transpose(1, 2).reshape(B, d)


def brute_force_trajectory(params: dict, cfg, e: np.ndarray, perturb_outside_window=None,
                           return_history: bool = False):
    """All s_t [B, T, d] for e [B, T, d], each recomputed from s*.

    ``perturb_outside_window``: optional torch.Generator; when given, before every
    self-attention call all stored keys/values older than the window get fresh noise
    (a pin of the mask itself: results must not change).
    ``return_history``: also return the full per-layer key/value history of the last target
    ([L, B, T, d] each).
    """
    P = {k: _t(v) for k, v in params.items()}
    E = _t(e)
    B, T, d = E.shape
    L, H, W = cfg.n_layers, cfg.n_heads, cfg.window
    km = torch.stack([E @ P["wmk"][g] for g in range(P["wmk"].shape[0])])
    vm = torch.stack([E @ P["wmv"][g] for g in range(P["wmv"].shape[0])])
    positions = torch.arange(1, T + 1)
    out = torch.empty(B, T, d, dtype=torch.float64)
    for target in range(1, T + 1):
        s = P["s_star"].expand(B, d).clone()
        hk = [[] for _ in range(L)]
        hv = [[] for _ in range(L)]
        for t in range(1, target + 1):
            e_t = E[:, t - 1]
            u = cfg.alpha * s
            g = torch.sigmoid(torch.cat([e_t, u], dim=-1) @ P["w_gate"] + P["b_gate"])
            h = g * e_t + (1 - g) * u
            for l in range(L):
                gam = P["gamma"][l]
                a = F.rms_norm(h, (d,), weight=gam[0], eps=cfg.eps)
                q, k, v = a @ P["wq"][l], a @ P["wk"][l], a @ P["wv"][l]
                hk[l].append(k)
                hv[l].append(v)
                pos = positions[:t]
                in_window = pos >= t - W + 1
                if perturb_outside_window is not None:
                    for j in range(t):
                        if not in_window[j]:
                            hk[l][j] = torch.randn(B, d, generator=perturb_outside_window,
                                                   dtype=torch.float64)
                            hv[l][j] = torch.randn(B, d, generator=perturb_outside_window,
                                                   dtype=torch.float64)
                o = _sdpa(q, torch.stack(hk[l], 1), torch.stack(hv[l], 1), in_window, H)
                h = h + o @ P["wo"][l]
                c = F.rms_norm(h, (d,), weight=gam[1], eps=cfg.eps)
                grp = 0 if cfg.n_groups == 1 else l
                prefix = positions <= t
                oc = _sdpa(c @ P["wcq"][l], km[grp], vm[grp], prefix, H)
                h = h + oc @ P["wco"][l]
                f = F.rms_norm(h, (d,), weight=gam[2], eps=cfg.eps)
                h = h + (F.silu(f @ P["w1"][l]) * (f @ P["w3"][l])) @ P["w2"][l]
            s = h
        out[:, target - 1] = s
    if return_history:
        hist_k = torch.stack([torch.stack(x, 1) for x in hk])
        hist_v = torch.stack([torch.stack(x, 1) for x in hv])
        return out.numpy(), hist_k.numpy(), hist_v.numpy()
    return out.numpy()
