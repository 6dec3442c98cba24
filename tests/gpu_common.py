"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the oracle on the same seeded inputs, optionally on sampled nodes."""
import numpy as np

from cartesian_tensor_product_amd import inputs

TOL = 1e-4   # max-abs error <= TOL * max|oracle| per output tensor


def f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def assert_close(name, got, want, floor=None):
    scale = np.abs(want).max()
    if floor is not None:
        scale = max(scale, floor)
    err = np.abs(np.asarray(got, dtype=np.float64) - want).max() if want.size else 0.0
    assert err <= TOL * scale, f"{name}: max err {err:.3e} > {TOL:g} * {scale:.3e}"
    return err / scale if scale else 0.0


class GpuConv:
    """One edge-convolution problem on the GPU (forward + VJP)."""

    def __init__(self, ranks, rc, d, channels, device="cuda", flags=0):
        import torch
        from cartesian_tensor_product_amd import flashcart as fc
        self.fc, self.torch = fc, torch
        self.N = d["pos"].shape[0]
        self.E = int(len(d["sender"]))
        self.C = channels
        self.desc = fc.conv_desc(self.N, self.E, channels, *ranks, rc, flags=flags)
        self.P, self.nin, self.nout = fc.fc_conv_layout(self.desc)
        self.graph = fc.DeviceGraph(d["rowptr"], d["sender"], self.N, device=device)
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
        self.pos, self.shift, self.x, self.W = t(d["pos"]), t(d.get("shift")), t(d["x"]), t(d["W"])
        self.g = t(d["g"]) if d.get("g") is not None else None
        self.ws = fc.workspace(fc.fc_edge_conv_workspace_bytes(self.desc, 1), device)
        self.device = device

    def fwd(self):
        z = self.torch.empty((self.N, self.nout, self.C), device=self.device)
        self.fc.fc_edge_conv_fwd(self.desc, self.graph, self.pos, self.shift, self.x, self.W, z)
        return z

    def vjp_vjp(self, v_x=None, v_pos=None, want=("g", "x", "pos"), g=None, v_W=None):
        """(g_hat, x_hat, pos_hat, radial_w_hat); entries not in ``want`` are None."""
        t = self.torch
        dv = lambda a: None if a is None else t.from_numpy(np.ascontiguousarray(a)).to(self.device)
        gh = t.empty((self.N, self.nout, self.C), device=self.device) if "g" in want else None
        xh = t.empty_like(self.x) if "x" in want else None
        ph = t.empty((self.N, 3), device=self.device) if "pos" in want else None
        Wh = t.empty_like(self.W) if "W" in want else None
        ws = self.fc.workspace(self.fc.fc_edge_conv_workspace_bytes(self.desc, 2), self.device)
        self.fc.fc_edge_conv_vjp_vjp(self.desc, self.graph, self.pos, self.shift, self.x, self.W,
                                     self.g if g is None else dv(g), dv(v_x), dv(v_pos), dv(v_W), gh, xh, ph, Wh,
                                     ws)
        return gh, xh, ph, Wh

    def vjp(self, g=None, want_x=True, want_pos=True, want_W=False):
        """(x_grad, pos_grad), or (x_grad, pos_grad, radial_w_grad) with want_W."""
        g = self.g if g is None else g
        xb = self.torch.empty_like(self.x) if want_x else None
        pb = self.torch.empty((self.N, 3), device=self.device) if want_pos else None
        Wb = self.torch.empty_like(self.W) if want_W else None
        self.fc.fc_edge_conv_vjp(self.desc, self.graph, self.pos, self.shift, self.x, self.W, g, xb, pb, Wb,
                                 self.ws)
        return (xb, pb, Wb) if want_W else (xb, pb)


def sample_edges(rowptr, sender, nodes):
    """Edge ids touching ``nodes`` (as receiver or as sender)."""
    nodes = np.asarray(nodes)
    recv = np.repeat(np.arange(len(rowptr) - 1), np.diff(rowptr))
    m = np.isin(recv, nodes) | np.isin(sender, nodes)
    return np.nonzero(m)[0]


def conv_inputs(name_or_params, ranks, rc=None, seed=None, n=None, k=None, box=None, C=None, with_vpos=False):
    from oracle import conv
    spec = conv.ConvSpec(*ranks, rc)
    d = inputs.edge_conv_inputs(seed, n, k, box, C, spec.n_in, spec.n_paths, spec.n_out, with_vpos=with_vpos)
    return spec, d
