"""Helpers shared by the GPU tests: device copies, library runs, error metrics."""
from __future__ import annotations

import numpy as np
import torch

import chunk_wise_weight_amd as ttt


def torch_dtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


class Layer:
    """A library handle plus the device copies of one workload's inputs."""

    def __init__(self, w, C=None, eta=None, G=0, max_batch=None):
        self.w = w
        self.dt = torch_dtype(w)
        self.C = w.C if C is None else C
        self.eta = w.eta if eta is None else eta
        self.h = ttt.ttt_init(dev(w.W_up, self.dt), dev(w.W_gate, self.dt), dev(w.W_down0, self.dt), self.C,
                              self.eta, max_batch=max_batch or w.B)
        if G:
            ttt.ttt_set_group_chunks(self.h, G)
        self.x = dev(w.x, self.dt)
        self.ids = torch.from_numpy(np.ascontiguousarray(w.ids)).cuda()
        self.E = dev(w.E_tgt, self.dt)

    def forward(self, x=None, ids=None):
        x = self.x if x is None else x
        ids = self.ids if ids is None else ids
        y, Wf = ttt.ttt_forward_chunked(self.h, x, ids, self.E, want_W_final=True)
        torch.cuda.synchronize()
        return y, Wf

    def forward_np(self, x=None, ids=None):
        y, Wf = self.forward(x, ids)
        return y.double().cpu().numpy(), Wf.double().cpu().numpy()


def max_rel(a, r):
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-300))


def rel_fro(a, r):
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.linalg.norm((a - r).ravel()) / max(np.linalg.norm(r.ravel()), 1e-300))
