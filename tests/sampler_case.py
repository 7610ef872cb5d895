"""Seeded inputs of a denoising run (stack + sampler) on the device and for
the oracle; shared by the GPU tests of the sampler and of the lazy profiles."""
from __future__ import annotations

import numpy as np
import torch

import masked_gqa_attention_action_amd as dmx
from masked_gqa_attention_action_amd import synth
from tests.helpers import device_weights, f64, oracle_weights, to_dev


class Case:
    """Seeded inputs of one sampler run, on the device and for the oracle."""

    def __init__(self, n_layers, n_steps, B, C, P, len_lo, len_hi, hole_p, seed, mod_table=False,
                 A=synth.ACTION_DIM):
        self.n_layers, self.n_steps, self.B, self.C, self.P = n_layers, n_steps, B, C, P
        wbits = [synth.layer_weights(seed + 100 + l) for l in range(n_layers)]
        self.rqs = [synth.make_request(seed + b, C, P, len_lo, len_hi, n_layers, hole_p) for b in range(B)]
        self.swbits = synth.sampler_weights(seed + 500, a=A)
        self.noise = synth.sampler_noise(seed + 600, B, C, a=A)
        self.A = self.noise.shape[2]
        print(f"sampler case: A={A} L={n_layers} steps={n_steps} B={B} C={C} P_b={P} "
              f"valid={[r.valid_len for r in self.rqs]} seed={seed}", flush=True)
        self.wbits = wbits
        self.wd = [device_weights(w) for w in wbits]
        self.kp = [to_dev(np.stack([r.k_pre[l] for r in self.rqs])) for l in range(n_layers)]
        self.vp = [to_dev(np.stack([r.v_pre[l] for r in self.rqs])) for l in range(n_layers)]
        self.mask = to_dev(np.stack([r.mask for r in self.rqs]), "raw")
        self.pos0 = to_dev(np.array([r.pos0 for r in self.rqs], np.int32), "raw")
        self.cond = torch.empty((n_steps, B, synth.H), dtype=torch.bfloat16, device="cuda")
        self.x = torch.empty((B, C, synth.H), dtype=torch.bfloat16, device="cuda")
        self.sw = dmx.pack_sampler_weights({k: to_dev(v) for k, v in self.swbits.items()})
        self.actions = torch.from_numpy(self.noise).cuda()
        self.traj = torch.empty((n_steps, B, C, self.A), dtype=torch.float32, device="cuda")
        self.stack = dmx.Stack(self.wd, self.kp, self.vp, self.mask, self.cond, self.pos0, self.x,
                               mod_table=mod_table)
        self.sampler = dmx.Sampler(self.stack, self.sw, self.actions, self.traj)

    def oracle_inputs(self):
        sw = {k: f64(v) for k, v in self.swbits.items()}
        layers = [oracle_weights(w) for w in self.wbits]
        return sw, layers

    def reset(self, noise=None):
        self.actions.copy_(torch.from_numpy(self.noise if noise is None else noise))
