"""A packed spectral MoE gate/up layer resident in device memory.

Host work is layout only: the library packer quantizes and packs each
linear type, and Phi_gate, Phi_up (din x r each) are stored transposed and
stacked as one 2r x din fp16 array so that one projection launch produces
z_gate and z_up together.  Everything the decode step computes runs in the
library's kernels.
"""
import numpy as np

from . import bitsmoe


class DeviceLayer:
    def __init__(self, phi_gate, phi_up, a_gate, a_up, p_gate, p_up, bits_gate, bits_up,
                 device="cuda", blobs=None):
        import torch
        self.E, self.r, self.dout = p_gate.shape
        self.din = phi_gate.shape[0]
        if blobs is None:
            blobs = (bitsmoe.pack(p_gate, a_gate, bits_gate), bitsmoe.pack(p_up, a_up, bits_up))
        self.host_blobs = blobs
        phi_t = np.concatenate([np.asarray(phi_gate, np.float16).T,
                                np.asarray(phi_up, np.float16).T], axis=0)
        self.phi_t = torch.from_numpy(np.ascontiguousarray(phi_t)).to(device)
        self.blob_gate = torch.from_numpy(blobs[0]).to(device)
        self.blob_up = torch.from_numpy(blobs[1]).to(device)
        self.device = device

    @classmethod
    def from_synth(cls, layer, device="cuda"):
        return cls(layer.phi["gate"], layer.phi["up"], layer.a["gate"], layer.a["up"],
                   layer.p["gate"], layer.p["up"], layer.bits["gate"], layer.bits["up"],
                   device=device)

    def workspace(self, T, k):
        import torch
        n = bitsmoe.moe_gateup_workspace_size(T, k, self.E, self.din, self.dout, self.r)
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=self.device)
        bitsmoe.workspace_init(ws)
        return ws

    def gateup(self, x, ids, h=None, ws=None, stream=None):
        import torch
        T, k = ids.shape
        if h is None:
            h = torch.empty((T, k, self.dout), dtype=torch.float32, device=self.device)
        if ws is None:
            ws = self.workspace(T, k)
        bitsmoe.moe_gateup(self.blob_gate, self.blob_up, self.phi_t, x, ids, self.E, self.dout,
                           self.r, h, ws, stream=stream)
        return h
