"""Device-buffer plumbing around the C ABI for one BitLinear weight.

`BitLinearWeight` owns the device buffers of one layer (mask, packed codes,
gamma, workspaces) and calls the library's entry points in the order the
method runs them: quantize_mask + pack once per training step (the mask is
recomputed every step) or once at load time for inference, then fwd / bwd
per batch.  torch is used for device memory and the stream only.
"""
import numpy as np
import torch

from . import bitlinear as bl


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class BitLinearWeight:
    def __init__(self, n_out, k, n=6, m=8, gamma_over=bl.BL_GAMMA_DENSE, device="cuda"):
        self.n_out, self.k, self.n, self.m = int(n_out), int(k), int(n), int(m)
        self.gamma_over = gamma_over
        nbytes = bl.bitlinear_packed_bytes(n_out, k, n, m)
        if nbytes == 0:
            raise ValueError(f"unsupported layer {n_out}x{k} {n}:{m}")
        self.mask = torch.empty(n_out * (k // 8), dtype=torch.uint8, device=device)
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.gamma = torch.empty(1, dtype=torch.float64, device=device)
        self.ws = torch.empty(bl.bitlinear_workspace_bytes(n_out, k), dtype=torch.uint8, device=device)
        self.device = device

    def quantize(self, W, wq=None, stream=None):
        """Mask + gamma (+ optional int8 codes), then pack."""
        bl.bitlinear_quantize_mask(W, self.n_out, self.k, self.n, self.m, self.gamma_over, self.mask,
                                   wq, self.gamma, self.ws, stream=stream)
        bl.bitlinear_pack(W, self.mask, self.gamma, self.n_out, self.k, self.n, self.m, self.packed,
                          stream=stream)

    def fwd_buffers(self, tokens):
        d = self.device
        ws_n = bl.bitlinear_fwd_workspace_bytes(tokens, self.k, self.n_out)
        return {
            "Y": torch.empty(tokens * self.n_out, dtype=torch.float32, device=d),
            "xq": torch.empty(tokens * self.k, dtype=torch.int8, device=d),
            "x_scale": torch.empty(max(tokens, 1), dtype=torch.float32, device=d)[:tokens],
            # zero-filled once: bitlinear_contract needs zero counters on entry
            # and leaves them zero (bitlinear_fwd clears them itself)
            "ws": torch.zeros(ws_n, dtype=torch.uint8, device=d) if ws_n else None,
        }

    def fwd(self, X, tokens, bufs=None, acc=None, stream=None):
        b = bufs if bufs is not None else self.fwd_buffers(tokens)
        bl.bitlinear_fwd(X, tokens, self.k, self.packed, self.n_out, self.n, self.m, self.gamma,
                         b["Y"], b["xq"], b["x_scale"], acc=acc, ws=b["ws"], stream=stream)
        return b

    def bwd_workspace(self, tokens):
        """Device scratch of the backward (bf16 operands of its products)."""
        n = bl.bitlinear_bwd_workspace_bytes(tokens, self.k, self.n_out)
        return torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)

    def bwd(self, dY, xq, x_scale, tokens, dX=True, dW=True, ws=None, stream=None):
        d = self.device
        gx = torch.empty(tokens * self.k, dtype=torch.float32, device=d) if dX else None
        gw = torch.empty(self.n_out * self.k, dtype=torch.float32, device=d) if dW else None
        if ws is None:
            ws = self.bwd_workspace(tokens)
        bl.bitlinear_bwd(dY, xq, x_scale, self.packed, self.gamma, tokens, self.k, self.n_out,
                         self.n, self.m, gx, gw, ws=ws, stream=stream)
        return gx, gw


class QuantGroup:
    """Grouped weight quantisation of several BitLinearWeight layers that
    share one N:M pattern and gamma mode: the plan (device descriptors) is
    built once for fixed (weight, layer) pairs, then each `run` recomputes
    every mask, gamma and packed block in three launches."""

    def __init__(self, pairs, stream=None):
        lws = [lw for lw, _ in pairs]
        if not lws:
            raise ValueError("QuantGroup needs at least one layer")
        n, m, go = lws[0].n, lws[0].m, lws[0].gamma_over
        if any((lw.n, lw.m, lw.gamma_over) != (n, m, go) for lw in lws):
            raise ValueError("all layers of a QuantGroup share n, m and gamma_over")
        self.n, self.m, self.gamma_over = n, m, go
        self.weights = [W for _, W in pairs]
        entries = [dict(W=W, mask=lw.mask, gamma=lw.gamma, packed=lw.packed, n_out=lw.n_out, k=lw.k)
                   for lw, W in pairs]
        self.items = bl.make_quant_items(entries, n, m)
        d = lws[0].device
        self.ws = torch.empty(max(bl.bitlinear_quant_group_workspace_bytes(self.items, len(entries)), 1),
                              dtype=torch.uint8, device=d)
        self.plan = torch.empty(bl.bitlinear_quant_group_plan_bytes(self.items, len(entries)),
                                dtype=torch.uint8, device=d)
        bl.bitlinear_quant_group_plan(self.items, len(entries), n, m, go, self.ws, self.plan, stream=stream)

    def run(self, stream=None):
        bl.bitlinear_quant_group(self.plan, self.n, self.m, self.gamma_over, stream=stream)


class LatentWeights:
    """binary32 latent weights of one layer and the bf16 copy the weight
    path reads; `update` applies one plain gradient step on the device."""

    def __init__(self, W_bf16, device="cuda"):
        self.W = W_bf16.contiguous().to(device)
        self.master = self.W.float().contiguous()

    def update(self, dW, lr, stream=None):
        bl.bitlinear_latent_update(self.master, dW, self.master.numel(), lr, self.W, stream=stream)


def dense_to_sparse(step, switch_step, n, m):
    """N:M pattern of a dense-to-sparse schedule: dense (8:8) before
    switch_step, n:m from it on."""
    return (8, 8) if step < switch_step else (n, m)
