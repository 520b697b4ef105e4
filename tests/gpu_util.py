"""Helpers for the GPU parity tests: device copies of synthetic inputs and the
per-row error metric (max over rows of ||y_gpu - y_ref|| / ||y_ref||)."""
import numpy as np
import torch

from precision_moe_expert_amd import binding, synth

ROW_TOL = 2e-2  # max relative L2 error per output row (bf16 output)


def dev(a: np.ndarray, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
        t = t.view(torch.bfloat16) if dtype == "bf16" else t
    elif a.dtype == np.uint8:
        t = torch.from_numpy(a)
    else:
        t = torch.from_numpy(a)
    return t.cuda()


class DevInputs:
    def __init__(self, li: synth.LayerInputs):
        c = li.cfg
        self.li = li
        self.x = dev(li.x, "bf16")
        self.logits = dev(li.logits)
        self.w13 = dev(li.w13)
        self.w2 = dev(li.w2)
        self.s13 = dev(li.s13)
        self.s2 = dev(li.s2)
        self.oft = dev(li.oft, "bf16") if li.oft is not None else None
        self.g13 = dev(li.g13) if li.g13 is not None else None
        self.g2 = dev(li.g2) if li.g2 is not None else None
        self.layer = binding.make_layer(c.T, c.H, c.I, c.E, c.k, c.fmt, oft=li.oft is not None)

    def forward(self, chunk=None, out=None, ws=None):
        c = self.li.cfg
        return binding.expert_forward(self.layer, self.x, self.logits, self.w13, self.w2, self.s13, self.s2,
                                      adapter=self.oft, chunk_experts=c.chunk if chunk is None else chunk,
                                      out=out, ws=ws, g13=self.g13, g2=self.g2)

    def forward_materialized(self, chunk=None, out=None, ws=None):
        c = self.li.cfg
        return binding.expert_forward_materialized(self.layer, self.x, self.logits, self.w13, self.w2, self.s13,
                                                   self.s2, adapter=self.oft,
                                                   chunk_experts=c.chunk if chunk is None else chunk, out=out, ws=ws,
                                                   g13=self.g13, g2=self.g2)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
