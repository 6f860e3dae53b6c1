"""Helpers for the GPU parity tests: device copies of the generator's arrays."""

import numpy as np
import torch

DEV = "cuda:0"


def bits_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


class DraftDev:
    """Device copies of a dsa_inputs.DraftInputs batch."""

    def __init__(self, d):
        self.d = d
        self.q_index = bits_to_dev(d.q_index_bits)
        self.w = to_dev(d.w)
        self.kidx = bits_to_dev(d.kidx_bits)
        self.bt = to_dev(d.block_table)
        self.row_len = to_dev(d.row_len)
        self.q = bits_to_dev(d.q_bits)                 # [G, B, H_q, D_qk]
        self.k = bits_to_dev(d.k_bits)
        self.v = self.k if d.v_bits is None else bits_to_dev(d.v_bits)

    @property
    def ld(self):
        return int(max(self.d.lens)) + self.d.G
