"""A torch.nn.Module over the C ABI: the MoE layer as a differentiable PyTorch op.

Buffer plumbing only.  The forward is one moe_layer_fwd call and the backward
one moe_layer_bwd call (plus moe_transpose_weights when a weight changed);
this module allocates their outputs, intermediates and workspaces with torch
and hands the pointers over.  Nothing here computes a step of the layer.

    layer = MoELayer(cfg)                 # cfg: any object with the moe_config fields
    y, aux = layer(x)                     # aux: GShard aux loss (one head), else None
    (loss_of(y) + 0.01 * aux).backward()  # gradients of x and every weight

The gradient reaching `aux` is the aux weight of moe_layer_bwd; reading it is
one device-to-host copy per backward.  The balancing bias (sel_bias buffer),
when enabled, steers selection only and is never trained by gradients;
`update_sel_bias(gamma)` applies moe_sel_bias_update with the last forward's
loads.
"""
import torch

from . import (MOE_LOGITS_COMPUTE_STORE, backward_workspace, moe_layer_bwd, moe_layer_fwd, moe_rows_upper_bound,
               moe_sel_bias_update, moe_transpose_weights, workspace)

_WEIGHTS = ("w_router", "router_bias", "w1", "w3", "w2", "ws1", "ws3", "ws2", "w_in", "w_out")


def _act_dtype(cfg):
    return torch.bfloat16 if cfg.act_dtype == 1 else torch.float32


class _MoEFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, layer, x, *params):
        cfg = layer.cfg
        W = dict(zip(_WEIGHTS, params))
        W["sel_bias"] = layer.sel_bias
        T, K, E = cfg.T, cfg.k_total, cfg.n_experts
        Rm = max(moe_rows_upper_bound(cfg), 1)
        adt = _act_dtype(cfg)
        dev = x.device
        e = lambda *s, dt=adt: torch.empty(*s, dtype=dt, device=dev)
        io = dict(logits=e(T, E, dt=torch.float32), logits_mode=MOE_LOGITS_COMPUTE_STORE,
                  topk_idx=e(T, K, dt=torch.int32), topk_w=e(T, K, dt=torch.float32), demand=e(E, dt=torch.int32),
                  counts=e(E, dt=torch.int32), offsets=e(E + 1, dt=torch.int32), row_of=e(T, K, dt=torch.int32),
                  src_of=e(Rm, dt=torch.int32), y_perm=e(Rm, cfg.d_head),
                  aux_loss=e(1, dt=torch.float32) if cfg.n_heads == 1 else None,
                  z=e(T, cfg.n_heads * cfg.d_head) if cfg.latent_proj else None,
                  o=e(T, cfg.n_heads * cfg.d_head) if cfg.latent_proj else None)
        y = torch.empty_like(x)
        moe_layer_fwd(cfg, W, x, y, io, layer._fwd_ws(dev))
        ctx.layer, ctx.io, ctx.W = layer, io, W
        ctx.save_for_backward(x)
        layer.last_io = io
        aux = io["aux_loss"] if io["aux_loss"] is not None else torch.zeros(1, device=dev)
        ctx.mark_non_differentiable(*([] if io["aux_loss"] is not None else [aux]))
        return y, aux

    @staticmethod
    def backward(ctx, dy, daux):
        layer, io, W = ctx.layer, ctx.io, ctx.W
        (x,) = ctx.saved_tensors
        cfg = layer.cfg
        aux_weight = 0.0
        if daux is not None and cfg.n_heads == 1:
            aux_weight = float(daux.reshape(-1)[0].item())
        G = layer._grads(x.device)
        moe_layer_bwd(cfg, W, layer._transposed(W), x, dy.contiguous(), aux_weight, io, G,
                      layer._bwd_ws(x.device))
        out = [None, G["dx"]]
        for name in _WEIGHTS:
            p = W[name]
            if p is None or not p.requires_grad:
                out.append(None)
                continue
            g = G[{"router_bias": "dbias"}.get(name, "d" + name)]
            out.append(g.to(p.dtype))
        return tuple(out)


class MoELayer(torch.nn.Module):
    """The MoE layer of `cfg` with its weights as parameters (N(0, 1/d_in) initialisation)."""

    def __init__(self, cfg, device="cuda", router_bias=None, sel_bias=None, seed=0):
        super().__init__()
        self.cfg = cfg
        adt = _act_dtype(cfg)
        rdt = torch.float32 if cfg.router_dtype == 0 else torch.bfloat16
        gen = torch.Generator(device="cpu").manual_seed(seed)
        E, dh, F, d, H = cfg.n_experts, cfg.d_head, cfg.d_ff, cfg.d_model, cfg.n_heads

        def param(shape, fan_in, dt):
            w = torch.randn(*shape, generator=gen) / fan_in ** 0.5
            return torch.nn.Parameter(w.to(dt).to(device))

        self.w_router = param((E, dh), dh, rdt)
        self.router_bias = None if router_bias is None else torch.nn.Parameter(
            torch.as_tensor(router_bias, dtype=torch.float32, device=device).clone())
        self.w1 = param((E, F, dh), dh, adt)
        self.w3 = param((E, F, dh), dh, adt) if cfg.act == 1 else None
        self.w2 = param((E, dh, F), F, adt)
        fs = cfg.n_shared * F
        self.ws1 = param((fs, d), d, adt) if fs else None
        self.ws3 = param((fs, d), d, adt) if (fs and cfg.act == 1) else None
        self.ws2 = param((d, fs), fs, adt) if fs else None
        self.w_in = param((H * dh, d), d, adt) if cfg.latent_proj else None
        self.w_out = param((d, H * dh), H * dh, adt) if cfg.latent_proj else None
        self.register_buffer("sel_bias", None if sel_bias is None else
                             torch.as_tensor(sel_bias, dtype=torch.float32, device=device).clone())
        self.last_io = None
        self._ws = {}
        self._wt = None
        self._wt_versions = None

    def weights(self):
        return {n: getattr(self, n) for n in _WEIGHTS}

    def forward(self, x):
        params = [getattr(self, n) for n in _WEIGHTS]
        y, aux = _MoEFunction.apply(self, x.contiguous(), *params)
        return y, (aux if self.cfg.n_heads == 1 else None)

    @torch.no_grad()
    def update_sel_bias(self, gamma=0.001):
        """One balancing-bias step from the last forward's per-expert loads."""
        if self.sel_bias is None or self.last_io is None:
            raise RuntimeError("no selection bias, or no forward yet")
        moe_sel_bias_update(self.cfg, self.last_io["demand"], self.sel_bias, gamma)

    # ------------------------------------------------------------ buffers
    def _fwd_ws(self, dev):
        if "fwd" not in self._ws:
            self._ws["fwd"] = workspace(self.cfg, dev)
        return self._ws["fwd"]

    def _bwd_ws(self, dev):
        if "bwd" not in self._ws:
            self._ws["bwd"] = backward_workspace(self.cfg, dev)
        return self._ws["bwd"]

    def _transposed(self, W):
        """Transposed weights for the backward, rebuilt when a weight has changed."""
        cfg = self.cfg
        versions = tuple((n, W[n]._version) for n in ("w1", "w3", "w2", "ws1", "ws3", "ws2", "w_in", "w_out")
                         if W[n] is not None)
        if self._wt is None or versions != self._wt_versions:
            adt = _act_dtype(cfg)
            dev = W["w1"].device
            E, dh, F, d = cfg.n_experts, cfg.d_head, cfg.d_ff, cfg.d_model
            m = 2 if cfg.act == 1 else 1
            fs = cfg.n_shared * F
            D = cfg.n_heads * dh
            e = lambda *s: torch.empty(*s, dtype=adt, device=dev)
            self._wt = dict(w13t=e(E, dh, m * F), w2t=e(E, F, dh), ws13t=e(d, m * fs) if fs else None,
                            ws2t=e(fs, d) if fs else None, w_in_t=e(d, D) if cfg.latent_proj else None,
                            w_out_t=e(D, d) if cfg.latent_proj else None)
            moe_transpose_weights(cfg, {k: v.detach() if v is not None else None for k, v in W.items()}, self._wt)
            self._wt_versions = versions
        return self._wt

    def _grads(self, dev):
        cfg = self.cfg
        adt = _act_dtype(cfg)
        E, dh, F, d = cfg.n_experts, cfg.d_head, cfg.d_ff, cfg.d_model
        fs = cfg.n_shared * F
        D = cfg.n_heads * dh
        e = lambda *s, dt=adt: torch.empty(*s, dtype=dt, device=dev)
        return dict(dx=e(cfg.T, d), dw_router=e(E, dh, dt=torch.float32), dbias=e(E, dt=torch.float32),
                    dw1=e(E, F, dh), dw3=e(E, F, dh) if cfg.act == 1 else None, dw2=e(E, dh, F),
                    dws1=e(fs, d) if fs else None, dws3=e(fs, d) if (fs and cfg.act == 1) else None,
                    dws2=e(d, fs) if fs else None, dw_in=e(D, d) if cfg.latent_proj else None,
                    dw_out=e(d, D) if cfg.latent_proj else None)
