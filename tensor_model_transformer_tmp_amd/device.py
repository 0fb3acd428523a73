"""Device-resident buffers of one TMP shard, allocated with torch and bound to
a liboases_shard context.  torch only allocates and copies here; all compute
is in the library's kernels."""
from __future__ import annotations

import numpy as np
import torch

from . import shard


def to_device(arr: np.ndarray, dtype: int, device) -> torch.Tensor:
    """Storage-form numpy array (float32, or uint16 bf16 bit patterns) -> device tensor."""
    if dtype == shard.BF16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def to_storage(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage-form numpy array (uint16 bits for bf16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceShard:
    """Allocates and binds every buffer of a step for ``inp`` (gen.ShardInputs)."""

    def __init__(self, inp, device="cuda", modes=("overlap_fine", "serial_fine", "serial_default",
                                                   "serial_norecompute"), streams=None):
        cfg = inp.cfg
        self.cfg, self.device = cfg, torch.device(device)
        tdt = torch.bfloat16 if cfg.dtype == shard.BF16 else torch.float32
        up = lambda a: to_device(a, cfg.dtype, self.device)
        L, N, h = cfg.n_layers, cfg.tokens, cfg.hidden
        self.x, self.dy = up(inp.x), up(inp.g)
        self.y = torch.zeros(N, h, dtype=tdt, device=self.device)
        self.dx = torch.zeros(N, h, dtype=tdt, device=self.device)
        self.ckpt = torch.zeros(L - 1, N, h, dtype=tdt, device=self.device) if L > 1 else None
        self.peers_fwd = up(inp.peers_fwd) if cfg.tmp_width > 1 else None
        self.peers_bwd = up(inp.peers_bwd) if cfg.tmp_width > 1 else None
        ws = max(shard.workspace_bytes(cfg, m) for m in modes)
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=self.device)
        self.params = []
        for l in range(L):
            self.params.append({
                "w_in": up(inp.w_in[l]), "b_in": up(inp.b_in[l]), "w_out": up(inp.w_out[l]),
                "dw_in": torch.zeros(cfg.n_in(l), h, dtype=torch.float32, device=self.device),
                "db_in": torch.zeros(cfg.n_in(l), dtype=torch.float32, device=self.device),
                "dw_out": torch.zeros(h, cfg.n_mid(l), dtype=torch.float32, device=self.device)})
            if getattr(cfg, "full_block", False):
                self.params[-1].update({
                    "ln_w": up(inp.ln_w[l]), "ln_b": up(inp.ln_b[l]),
                    "dln_w": torch.zeros(h, dtype=torch.float32, device=self.device),
                    "dln_b": torch.zeros(h, dtype=torch.float32, device=self.device)})
        self.ctx = shard.ShardContext(cfg)
        self.ctx.bind({"x": self.x, "y": self.y, "dy": self.dy, "dx": self.dx, "ckpt": self.ckpt,
                       "peers_fwd": self.peers_fwd, "peers_bwd": self.peers_bwd,
                       "workspace": self.workspace}, self.params)
        if streams is None:
            streams = (torch.cuda.Stream(self.device), torch.cuda.Stream(self.device))
        self.compute, self.side = streams
        self.ctx.set_streams(self.compute, self.side)

    def step(self, mode="overlap_fine", use_graph=False, sync=True):
        self.ctx.schedule_step(mode, use_graph)
        if sync:
            self.ctx.sync()

    def results(self) -> dict:
        """Storage-form host copies of Y, dX and the float32 gradients."""
        torch.cuda.synchronize(self.device)
        out = {"Y": to_storage(self.y), "dX": to_storage(self.dx), "grads": []}
        names = ("dw_in", "db_in", "dw_out") + (("dln_w", "dln_b") if getattr(self.cfg, "full_block", False) else ())
        for p in self.params:
            out["grads"].append({k: p[k].cpu().numpy() for k in names})
        return out

    def close(self):
        self.ctx.close()
