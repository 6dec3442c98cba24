"""Thin Python binding of libflashcart.so (ctypes).

Every function has the name of the C entry point it wraps and only marshals
arguments: torch tensors become device pointers, the stream defaults to
torch's current stream, and a non-OK status raises ``FlashCartError``.  All
computation happens in the library's HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashcart.so")

FC_OK, FC_ERR_INVALID_ARGUMENT, FC_ERR_UNSUPPORTED, FC_ERR_WORKSPACE, FC_ERR_HIP = range(5)
FC_LADDER_FULL, FC_LADDER_PATH_REDUCED = 0, 1
FC_CONV_ALL_PARITIES = 1   # descriptor flag: every triangle-allowed path (odd J too)
FC_CONV_SUM_PATHS = 2      # descriptor flag: outputs of the paths of each rank summed
FC_CONV_MLP_MATERIALIZE = 4  # descriptor flag: radial-network calls store w [E][P][C] instead of fusing it
FC_CONV_MLP_FUSE = 8         # descriptor flag: radial-network calls form w in the convolution's lanes


class FlashCartError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


class ConvDesc(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("n_edges", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("l_in", ctypes.c_int32), ("l_edge", ctypes.c_int32), ("l_out", ctypes.c_int32),
                ("n_basis", ctypes.c_int32), ("r_cut", ctypes.c_float), ("flags", ctypes.c_uint32)]


class Graph(ctypes.Structure):
    _fields_ = [("rowptr", ctypes.c_void_p), ("sender", ctypes.c_void_p), ("receiver", ctypes.c_void_p),
                ("t_rowptr", ctypes.c_void_p), ("t_edge", ctypes.c_void_p)]


class LadderDesc(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("channels", ctypes.c_int32), ("l_a", ctypes.c_int32),
                ("l_prod", ctypes.c_int32), ("l_out", ctypes.c_int32), ("order", ctypes.c_int32),
                ("variant", ctypes.c_int32)]


class NormDesc(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("channels", ctypes.c_int32), ("l_max", ctypes.c_int32),
                ("eps", ctypes.c_float)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_PD = ctypes.POINTER(ConvDesc)
_PL = ctypes.POINTER(LadderDesc)
_PG = ctypes.POINTER(Graph)
_PN = ctypes.POINTER(NormDesc)
_PI = ctypes.POINTER(ctypes.c_int32)
_PSZ = ctypes.POINTER(ctypes.c_size_t)

_SIGS = {
    "fc_status_string": (ctypes.c_char_p, [_I]),
    "fc_last_error_message": (ctypes.c_char_p, []),
    "fc_abi_version": (_I, []),
    "fc_conv_layout": (_I, [_PD, _PI, _PI, _PI]),
    "fc_conv_path": (_I, [_PD, _I, _PI, _PI, _PI]),
    "fc_graph_transpose_workspace_bytes": (_SZ, [_I]),
    "fc_graph_transpose": (_I, [_I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_graph_validate": (_I, [_I, _I, _PI, _PI]),
    "fc_edge_conv_workspace_bytes": (_SZ, [_PD, _I]),
    "fc_edge_conv_fwd": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _P]),
    "fc_edge_conv_vjp": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_edge_conv_vjp_noalloc": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "fc_edge_conv_vjp_vjp": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_edge_conv_fwd_w": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _P]),
    "fc_edge_conv_vjp_w": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_edge_conv_vjp_vjp_w": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_ladder_layout": (_I, [_PL, _PSZ, _PSZ]),
    "fc_ladder_workspace_bytes": (_SZ, [_PL, _I]),
    "fc_ladder_weight_block": (_I, [_PL, _I, _PSZ, _PI, _PI, _PI]),
    "fc_node_ladder_fwd": (_I, [_PL, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_node_ladder_vjp": (_I, [_PL, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_node_ladder_vjp_vjp": (_I, [_PL, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_radial_mlp_weight_floats": (_SZ, [_PD]),
    "fc_edge_conv_mlp_workspace_bytes": (_SZ, [_PD, _I]),
    "fc_radial_mlp": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_edge_conv_mlp_fwd": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_edge_conv_mlp_vjp": (_I, [_PD, _PG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_rms_norm_fwd": (_I, [_PN, _P, _P, _P, _P, _P]),
    "fc_rms_norm_workspace_bytes": (_SZ, [_PN]),
    "fc_rms_norm_vjp": (_I, [_PN, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "fc_message_block_weight_floats": (_SZ, [_PD, _PL]),
    "fc_message_block_workspace_bytes": (_SZ, [_PD, _PL]),
    "fc_message_block_energy_forces": (_I, [_PD, _PG, _P, _P, _P, _PL, _P, ctypes.c_float, ctypes.c_float, _P, _P,
                                            _P, _P, _SZ, _P]),
    "fc_block_workspace_bytes": (_SZ, [_PD, _PL]),
    "fc_block_energy_forces": (_I, [_PD, _PG, _P, _P, _P, _P, _PL, _P, ctypes.c_float, _P, _P, _P, _P, _SZ, _P]),
}


def lib() -> ctypes.CDLL:
    """Loads libflashcart.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -m cartesian_tensor_product_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().fc_status_string(s).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return str(s)


def _check(status: int) -> None:
    if status != FC_OK:
        raise FlashCartError(status, lib().fc_last_error_message().decode())


def _ptr(t, dtype=None):
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected dtype {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _f32(t):
    import torch
    return _ptr(t, torch.float32)


def _i32(t):
    import torch
    return _ptr(t, torch.int32)


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def conv_desc(n_nodes, n_edges, channels, l_in, l_edge, l_out, r_cut, n_basis=8, flags=0) -> ConvDesc:
    return ConvDesc(n_nodes, n_edges, channels, l_in, l_edge, l_out, n_basis, r_cut, flags)


def norm_desc(n_nodes, channels, l_max, eps) -> NormDesc:
    return NormDesc(n_nodes, channels, l_max, eps)


def ladder_desc(n_nodes, channels, l_a, l_prod, l_out, order, variant) -> LadderDesc:
    return LadderDesc(n_nodes, channels, l_a, l_prod, l_out, order, variant)


# ------------------------------------------------------------------ layout --

def fc_abi_version() -> int:
    return lib().fc_abi_version()


def fc_conv_layout(d: ConvDesc):
    p, i, o = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().fc_conv_layout(ctypes.byref(d), ctypes.byref(p), ctypes.byref(i), ctypes.byref(o)))
    return p.value, i.value, o.value


def fc_conv_path(d: ConvDesc, i: int):
    a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().fc_conv_path(ctypes.byref(d), i, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def fc_graph_validate(n_nodes: int, n_edges: int, rowptr, sender) -> None:
    """Host arrays (numpy int32)."""
    import numpy as np
    rp = np.ascontiguousarray(rowptr, dtype=np.int32)
    sd = np.ascontiguousarray(sender, dtype=np.int32)
    _check(lib().fc_graph_validate(n_nodes, n_edges, rp.ctypes.data_as(_PI), sd.ctypes.data_as(_PI)))


def fc_edge_conv_workspace_bytes(d: ConvDesc, op: int) -> int:
    return lib().fc_edge_conv_workspace_bytes(ctypes.byref(d), op)


def fc_ladder_layout(d: LadderDesc):
    w, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().fc_ladder_layout(ctypes.byref(d), ctypes.byref(w), ctypes.byref(s)))
    return w.value, s.value


def fc_ladder_workspace_bytes(d: LadderDesc, op: int) -> int:
    return lib().fc_ladder_workspace_bytes(ctypes.byref(d), op)


def fc_ladder_weight_block(d: LadderDesc, i: int):
    """(offset, rows, cols, kind) of block i of the flat weight buffer."""
    off, r, c, k = ctypes.c_size_t(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().fc_ladder_weight_block(ctypes.byref(d), i, ctypes.byref(off), ctypes.byref(r), ctypes.byref(c),
                                        ctypes.byref(k)))
    return off.value, r.value, c.value, k.value


def ladder_weight_blocks(d: LadderDesc):
    out, i = [], 0
    while True:
        try:
            out.append(fc_ladder_weight_block(d, i))
        except FlashCartError:
            return out
        i += 1


# ------------------------------------------------------------------- graph --

def fc_graph_transpose(n_nodes, n_edges, rowptr, sender, receiver, t_rowptr, t_edge, workspace, stream=None):
    _check(lib().fc_graph_transpose(n_nodes, n_edges, _i32(rowptr), _i32(sender), _i32(receiver),
                                    _i32(t_rowptr), _i32(t_edge), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))


class DeviceGraph:
    """Receiver-sorted CSR plus its sender-sorted transpose, on the GPU.

    Holds the int32 device tensors and the ``Graph`` struct passed to the
    convolution calls.  The transpose is built by ``fc_graph_transpose``.
    """

    def __init__(self, rowptr, sender, n_nodes: int, device="cuda", stream=None):
        import numpy as np
        import torch
        # the device calls do not check graph contents: validate the host
        # copy (an out-of-range sender would make the transpose write out of
        # bounds)
        h_rowptr = np.ascontiguousarray(torch.as_tensor(rowptr).cpu().numpy(), dtype=np.int32)
        h_sender = np.ascontiguousarray(torch.as_tensor(sender).cpu().numpy(), dtype=np.int32)
        if h_rowptr.shape != (n_nodes + 1,):
            raise FlashCartError(FC_ERR_INVALID_ARGUMENT,
                                 f"rowptr has {h_rowptr.size} entries, expected n_nodes + 1 = {n_nodes + 1}")
        fc_graph_validate(n_nodes, int(h_sender.size), h_rowptr, h_sender)
        self.n_nodes = n_nodes
        self.rowptr = torch.as_tensor(rowptr, dtype=torch.int32, device=device).contiguous()
        self.sender = torch.as_tensor(sender, dtype=torch.int32, device=device).contiguous()
        self.n_edges = int(self.sender.numel())
        E = max(self.n_edges, 1)
        self.receiver = torch.empty(E, dtype=torch.int32, device=device)
        self.t_rowptr = torch.empty(n_nodes + 1, dtype=torch.int32, device=device)
        self.t_edge = torch.empty(E, dtype=torch.int32, device=device)
        nbytes = lib().fc_graph_transpose_workspace_bytes(n_nodes)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        sender_t = self.sender if self.n_edges else torch.zeros(1, dtype=torch.int32, device=device)
        fc_graph_transpose(n_nodes, self.n_edges, self.rowptr, sender_t, self.receiver, self.t_rowptr,
                           self.t_edge, ws, stream)
        self._ws = ws
        self.struct = Graph(self.rowptr.data_ptr(), sender_t.data_ptr(), self.receiver.data_ptr(),
                            self.t_rowptr.data_ptr(), self.t_edge.data_ptr())
        self._sender_t = sender_t


# ---------------------------------------------------------- edge convolution --

def fc_edge_conv_fwd(d: ConvDesc, graph: DeviceGraph, pos, shift, x, radial_w, z, stream=None):
    _check(lib().fc_edge_conv_fwd(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift), _f32(x),
                                  _f32(radial_w), _f32(z), _stream(stream)))


def fc_edge_conv_vjp(d: ConvDesc, graph: DeviceGraph, pos, shift, x, radial_w, g_z, x_grad, pos_grad,
                     radial_w_grad, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_edge_conv_vjp(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift), _f32(x),
                                  _f32(radial_w), _f32(g_z), _f32(x_grad), _f32(pos_grad), _f32(radial_w_grad),
                                  _ptr(workspace), nbytes, _stream(stream)))


def fc_edge_conv_vjp_noalloc(d: ConvDesc, graph: DeviceGraph, pos, shift, x, radial_w, g_z, x_grad, pos_grad,
                             radial_w_grad, stream=None):
    """fc_edge_conv_vjp with the library's own per-GPU scratch (no workspace)."""
    _check(lib().fc_edge_conv_vjp_noalloc(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift),
                                          _f32(x), _f32(radial_w), _f32(g_z), _f32(x_grad), _f32(pos_grad),
                                          _f32(radial_w_grad), _stream(stream)))


def fc_edge_conv_fwd_w(d: ConvDesc, graph: DeviceGraph, pos, shift, x, w, z, stream=None):
    _check(lib().fc_edge_conv_fwd_w(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift), _f32(x),
                                    _f32(w), _f32(z), _stream(stream)))


def fc_edge_conv_vjp_w(d: ConvDesc, graph: DeviceGraph, pos, shift, x, w, g_z, x_grad, pos_grad, w_grad,
                       workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_edge_conv_vjp_w(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift), _f32(x),
                                    _f32(w), _f32(g_z), _f32(x_grad), _f32(pos_grad), _f32(w_grad), _ptr(workspace),
                                    nbytes, _stream(stream)))


def fc_edge_conv_vjp_vjp(d: ConvDesc, graph: DeviceGraph, pos, shift, x, radial_w, g_z, v_x, v_pos, v_radial_w,
                         g_hat, x_hat, pos_hat, radial_w_hat, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_edge_conv_vjp_vjp(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift),
                                      _f32(x), _f32(radial_w), _f32(g_z), _f32(v_x), _f32(v_pos),
                                      _f32(v_radial_w), _f32(g_hat), _f32(x_hat), _f32(pos_hat),
                                      _f32(radial_w_hat), _ptr(workspace), nbytes, _stream(stream)))


def fc_edge_conv_vjp_vjp_w(d: ConvDesc, graph: DeviceGraph, pos, shift, x, w, g_z, v_x, v_pos, v_w,
                           g_hat, x_hat, pos_hat, w_hat, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_edge_conv_vjp_vjp_w(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift),
                                        _f32(x), _f32(w), _f32(g_z), _f32(v_x), _f32(v_pos), _f32(v_w),
                                        _f32(g_hat), _f32(x_hat), _f32(pos_hat), _f32(w_hat), _ptr(workspace),
                                        nbytes, _stream(stream)))


# ------------------------------------------------------------------ ladder --

def fc_node_ladder_fwd(d: LadderDesc, A, weights, z, saved, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_node_ladder_fwd(ctypes.byref(d), _f32(A), _f32(weights), _f32(z), _f32(saved),
                                    _ptr(workspace), nbytes, _stream(stream)))


def fc_node_ladder_vjp(d: LadderDesc, A, weights, saved, g_z, A_grad, weights_grad, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_node_ladder_vjp(ctypes.byref(d), _f32(A), _f32(weights), _f32(saved), _f32(g_z),
                                    _f32(A_grad), _f32(weights_grad), _ptr(workspace), nbytes, _stream(stream)))


# ------------------------------------------------------------------ radial --

def fc_radial_mlp_weight_floats(d: ConvDesc) -> int:
    return lib().fc_radial_mlp_weight_floats(ctypes.byref(d))


def fc_edge_conv_mlp_workspace_bytes(d: ConvDesc, op: int) -> int:
    return lib().fc_edge_conv_mlp_workspace_bytes(ctypes.byref(d), op)


def fc_radial_mlp(d: ConvDesc, graph: DeviceGraph, pos, shift, mlp_w, w, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_radial_mlp(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift), _f32(mlp_w),
                               _f32(w), _ptr(workspace), nbytes, _stream(stream)))


def fc_edge_conv_mlp_fwd(d: ConvDesc, graph: DeviceGraph, pos, shift, x, mlp_w, z, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_edge_conv_mlp_fwd(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift), _f32(x),
                                      _f32(mlp_w), _f32(z), _ptr(workspace), nbytes, _stream(stream)))


def fc_edge_conv_mlp_vjp(d: ConvDesc, graph: DeviceGraph, pos, shift, x, mlp_w, g_z, x_grad, pos_grad, mlp_w_grad,
                         workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_edge_conv_mlp_vjp(ctypes.byref(d), ctypes.byref(graph.struct), _f32(pos), _f32(shift), _f32(x),
                                      _f32(mlp_w), _f32(g_z), _f32(x_grad), _f32(pos_grad), _f32(mlp_w_grad),
                                      _ptr(workspace), nbytes, _stream(stream)))


# -------------------------------------------------------------------- norm --

def fc_rms_norm_fwd(d: NormDesc, x, gamma, y, inv_scale, stream=None):
    _check(lib().fc_rms_norm_fwd(ctypes.byref(d), _f32(x), _f32(gamma), _f32(y), _f32(inv_scale),
                                 _stream(stream)))


def fc_rms_norm_workspace_bytes(d: NormDesc) -> int:
    return lib().fc_rms_norm_workspace_bytes(ctypes.byref(d))


def fc_rms_norm_vjp(d: NormDesc, x, gamma, inv_scale, g_y, x_grad, gamma_grad, workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_rms_norm_vjp(ctypes.byref(d), _f32(x), _f32(gamma), _f32(inv_scale), _f32(g_y), _f32(x_grad),
                                 _f32(gamma_grad), _ptr(workspace), nbytes, _stream(stream)))


def fc_node_ladder_vjp_vjp(d: LadderDesc, A, weights, saved, g_z, v_A, v_weights, g_hat, A_hat, weights_hat,
                           workspace, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_node_ladder_vjp_vjp(ctypes.byref(d), _f32(A), _f32(weights), _f32(saved), _f32(g_z), _f32(v_A),
                                        _f32(v_weights), _f32(g_hat), _f32(A_hat), _f32(weights_hat),
                                        _ptr(workspace), nbytes, _stream(stream)))


# ------------------------------------------------------------------- block --

def fc_block_workspace_bytes(conv: ConvDesc, lad: LadderDesc) -> int:
    return lib().fc_block_workspace_bytes(ctypes.byref(conv), ctypes.byref(lad))


def fc_block_energy_forces(conv: ConvDesc, graph: DeviceGraph, pos, shift, x, radial_w, lad: LadderDesc, ladder_w,
                           conv_scale: float, energy, e_atom, forces, workspace, stream=None):
    import torch
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_block_energy_forces(ctypes.byref(conv), ctypes.byref(graph.struct), _f32(pos), _f32(shift),
                                        _f32(x), _f32(radial_w), ctypes.byref(lad), _f32(ladder_w),
                                        ctypes.c_float(conv_scale), _ptr(energy, torch.float64), _f32(e_atom),
                                        _f32(forces), _ptr(workspace), nbytes, _stream(stream)))


def workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def fc_message_block_weight_floats(conv: ConvDesc, lad: LadderDesc) -> int:
    return lib().fc_message_block_weight_floats(ctypes.byref(conv), ctypes.byref(lad))


def fc_message_block_workspace_bytes(conv: ConvDesc, lad: LadderDesc) -> int:
    return lib().fc_message_block_workspace_bytes(ctypes.byref(conv), ctypes.byref(lad))


def fc_message_block_energy_forces(conv: ConvDesc, graph: DeviceGraph, pos, shift, h0, lad: LadderDesc, weights,
                                   conv_scale: float, eps: float, energy, e_atom, forces, workspace, stream=None):
    import torch
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fc_message_block_energy_forces(ctypes.byref(conv), ctypes.byref(graph.struct), _f32(pos),
                                                _f32(shift), _f32(h0), ctypes.byref(lad), _f32(weights),
                                                ctypes.c_float(conv_scale), ctypes.c_float(eps),
                                                _ptr(energy, torch.float64), _f32(e_atom), _f32(forces),
                                                _ptr(workspace), nbytes, _stream(stream)))
