"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point declared in include/flashcart.h, and its layout queries and
argument checks behave as documented."""
import os
import re

import numpy as np
import pytest

from cartesian_tensor_product_amd import flashcart as fc
from oracle import conv, ladder

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(fc.LIB_PATH), reason="libflashcart.so not built")


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "flashcart.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fc_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 16
    L = fc.lib()
    for n in names:
        assert hasattr(L, n), n
    out = os.popen(f"nm -D --defined-only {fc.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def test_abi_version_and_status_strings():
    assert fc.fc_abi_version() == 3
    L = fc.lib()
    assert L.fc_status_string(0) == b"FC_OK"
    assert L.fc_status_string(3) == b"FC_ERR_WORKSPACE"


@pytest.mark.parametrize("ranks,allp", [((1, 1, 1), False), ((2, 2, 2), False), ((3, 3, 3), False),
                                        ((4, 4, 4), False), ((5, 5, 5), False), ((0, 3, 3), False),
                                        ((2, 3, 3), False), ((1, 1, 1), True), ((2, 2, 2), True),
                                        ((3, 3, 3), True), ((4, 4, 4), True)])
def test_layout_and_path_order_match_oracle(ranks, allp):
    spec = conv.ConvSpec(*ranks, 5.0, all_parities=allp)
    d = fc.conv_desc(10, 20, 16, *ranks, 5.0, flags=fc.FC_CONV_ALL_PARITIES if allp else 0)
    P, nin, nout = fc.fc_conv_layout(d)
    assert (P, nin, nout) == (spec.n_paths, spec.n_in, spec.n_out)
    assert [fc.fc_conv_path(d, i) for i in range(P)] == spec.paths
    with pytest.raises(fc.FlashCartError):
        fc.fc_conv_path(d, P)


@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (3, 3, 3), (4, 4, 4)])
def test_summed_layout_matches_oracle(ranks):
    """FC_CONV_SUM_PATHS: one 2L+1-row block per output rank; the path order
    (the order of the radial weights) is that of the separate layout."""
    spec = conv.ConvSpec(*ranks, 5.0, sum_paths=True)
    d = fc.conv_desc(10, 20, 16, *ranks, 5.0, flags=fc.FC_CONV_SUM_PATHS)
    P, nin, nout = fc.fc_conv_layout(d)
    assert (P, nin, nout) == (spec.n_paths, spec.n_in, spec.n_out) == (P, nin, (ranks[2] + 1) ** 2)
    assert [fc.fc_conv_path(d, i) for i in range(P)] == spec.paths


@pytest.mark.parametrize("bad,status", [
    (dict(n_nodes=0), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(n_edges=-1), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(channels=0), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(channels=300), fc.FC_ERR_UNSUPPORTED),
    (dict(l_in=6), fc.FC_ERR_UNSUPPORTED),
    (dict(l_in=5, l_edge=5, l_out=4), fc.FC_ERR_UNSUPPORTED),
    (dict(l_in=-1), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(n_basis=6), fc.FC_ERR_UNSUPPORTED),
    (dict(r_cut=0.0), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(r_cut=float("inf")), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(flags=16), fc.FC_ERR_UNSUPPORTED),
    (dict(flags=12), fc.FC_ERR_INVALID_ARGUMENT),                        # fuse and materialise
    (dict(flags=1, l_in=0, l_edge=2, l_out=2), fc.FC_ERR_UNSUPPORTED),   # not instantiated
    (dict(flags=2, l_in=0, l_edge=2, l_out=2), fc.FC_ERR_UNSUPPORTED),   # not instantiated
    (dict(flags=3), fc.FC_ERR_UNSUPPORTED),                             # summed + all parities
])
def test_descriptor_errors(bad, status):
    kw = dict(n_nodes=4, n_edges=8, channels=8, l_in=1, l_edge=1, l_out=1, r_cut=5.0, n_basis=8, flags=0)
    kw.update(bad)
    d = fc.conv_desc(**kw)
    with pytest.raises(fc.FlashCartError) as ei:
        fc.fc_conv_layout(d)
    assert ei.value.status == status
    # calls fail on the host before anything touches a GPU
    assert fc.fc_edge_conv_workspace_bytes(d, 1) == 0


def test_null_pointers_rejected_before_launch():
    d = fc.conv_desc(4, 8, 8, 1, 1, 1, 5.0)
    g = fc.Graph()
    L = fc.lib()
    import ctypes
    st = L.fc_edge_conv_fwd(ctypes.byref(d), ctypes.byref(g), None, None, None, None, None, None)
    assert st == fc.FC_ERR_INVALID_ARGUMENT
    assert b"rowptr" in L.fc_last_error_message()
    st = L.fc_edge_conv_vjp(ctypes.byref(d), ctypes.byref(g), None, None, None, None, None, None, None, None,
                            None, 0, None)
    assert st == fc.FC_ERR_INVALID_ARGUMENT


def test_graph_validate():
    fc.fc_graph_validate(3, 4, [0, 2, 3, 4], [1, 2, 0, 1])
    for rp, sd in [([1, 2, 3, 4], [1, 2, 0, 1]), ([0, 3, 2, 4], [1, 2, 0, 1]), ([0, 2, 3, 5], [1, 2, 0, 1]),
                   ([0, 2, 3, 4], [1, 2, 0, 3])]:
        with pytest.raises(fc.FlashCartError) as ei:
            fc.fc_graph_validate(3, 4, rp, sd)
        assert ei.value.status == fc.FC_ERR_INVALID_ARGUMENT


def test_device_graph_rejects_bad_graph_before_upload():
    """The device calls trust the graph; the binding validates the host copy
    first (an out-of-range sender, a short rowptr)."""
    for rp, sd, n in [([0, 2, 3, 4], [1, 2, 0, 3], 3), ([0, 2, 3], [1, 2, 0], 3)]:
        with pytest.raises(fc.FlashCartError) as ei:
            fc.DeviceGraph(np.array(rp, np.int32), np.array(sd, np.int32), n, device="cpu")
        assert ei.value.status == fc.FC_ERR_INVALID_ARGUMENT


def test_large_node_arrays_are_accepted():
    """Node arrays past 2 GiB (rank 4, 128 channels, 20 000 nodes: g is
    2.36 GB) are within the kernels' 64-bit offsets, so the descriptor and
    the workspace queries accept them."""
    d = fc.conv_desc(20000, 80000, 128, 4, 4, 4, 5.0)
    P, nin, nout = fc.fc_conv_layout(d)
    assert 20000 * nout * 128 * 4 > 2 ** 31
    assert fc.fc_edge_conv_workspace_bytes(d, 1) > 0
    assert fc.fc_edge_conv_workspace_bytes(d, 2) > 20000 * nout * 128 * 4


def test_ladder_row_index_limit():
    """The ladder's GEMM row index n (2l + 1) + c must stay below 2^26."""
    ok = fc.ladder_desc(7_000_000, 32, 4, 4, 4, 2, fc.FC_LADDER_PATH_REDUCED)
    fc.fc_ladder_layout(ok)
    big = fc.ladder_desc(7_500_000, 32, 4, 4, 4, 2, fc.FC_LADDER_PATH_REDUCED)
    with pytest.raises(fc.FlashCartError) as ei:
        fc.fc_ladder_layout(big)
    assert ei.value.status == fc.FC_ERR_UNSUPPORTED


def test_workspace_sizes():
    d = fc.conv_desc(1024, 131072, 128, 2, 2, 2, 5.0)
    assert fc.fc_edge_conv_workspace_bytes(d, 0) == 0
    assert fc.fc_edge_conv_workspace_bytes(d, 1) >= 131072 * 3 * 4


def test_vjp_vjp_workspace_holds_weight_cotangent_terms():
    """Op 2 adds room for the forward and VJP taken with the weight
    cotangent as weights: [N][out_rows][C], [N][in_rows][C] and [N][3]."""
    d = fc.conv_desc(1024, 131072, 128, 2, 2, 2, 5.0)
    P, nin, nout = fc.fc_conv_layout(d)
    w1 = fc.fc_edge_conv_workspace_bytes(d, 1)
    w2 = fc.fc_edge_conv_workspace_bytes(d, 2)
    assert w2 >= w1 + 4 * 1024 * 128 * (nout + nin) + 4 * 1024 * 3


@pytest.mark.parametrize("bad,status", [
    (dict(n_nodes=0), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(channels=0), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(channels=513), fc.FC_ERR_UNSUPPORTED),
    (dict(l_max=-1), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(l_max=6), fc.FC_ERR_UNSUPPORTED),
    (dict(eps=-1.0), fc.FC_ERR_INVALID_ARGUMENT),
    (dict(eps=float("nan")), fc.FC_ERR_INVALID_ARGUMENT),
])
def test_norm_descriptor_errors(bad, status):
    """The RMS norm rejects bad descriptors on the host (no GPU call)."""
    kw = dict(n_nodes=4, channels=8, l_max=2, eps=1e-5)
    kw.update(bad)
    d = fc.norm_desc(**kw)
    assert fc.fc_rms_norm_workspace_bytes(d) == 0
    with pytest.raises(fc.FlashCartError) as ei:
        fc.fc_rms_norm_fwd(d, None, None, None, None, stream=0)
    assert ei.value.status == status


def test_norm_workspace_size():
    d = fc.norm_desc(4096, 128, 3, 1e-5)
    assert fc.fc_rms_norm_workspace_bytes(d) == 1024 * 4 * 128 * 4
    d = fc.norm_desc(10, 16, 1, 0.0)
    assert fc.fc_rms_norm_workspace_bytes(d) == 3 * 2 * 16 * 4


def test_ladder_vjp_vjp_workspace():
    """Op 2 (VJP-of-VJP) holds four product buffers, four states and order - 1
    tangent states; the path-reduced ladder also four output-sized sums."""
    full = fc.ladder_desc(4096, 128, 3, 3, 3, 4, fc.FC_LADDER_FULL)
    red = fc.ladder_desc(4096, 128, 3, 3, 3, 4, fc.FC_LADDER_PATH_REDUCED)
    st = 4096 * 16 * 128 * 4
    assert fc.fc_ladder_workspace_bytes(full, 2) >= 4 * 4096 * 99 * 128 * 4 + 7 * st
    assert fc.fc_ladder_workspace_bytes(red, 2) >= 4 * 4096 * 99 * 128 * 4 + 7 * st + 4 * st


def test_message_block_weight_count_matches_oracle():
    from oracle import conv, ladder, model
    for order, var in ((3, "reduced"), (5, "full")):
        cspec = conv.ConvSpec(0, 3, 3, 5.0)
        lspec = ladder.LadderSpec(3, 3, 0, order, var, 32)
        n = sum(int(np.prod(s)) for _, s in model.block_weight_shapes(32, 3, cspec.n_paths, lspec))
        cd = fc.conv_desc(216, 1000, 32, 0, 3, 3, 5.0)
        ld = fc.ladder_desc(216, 32, 3, 3, 0, order, fc.FC_LADDER_FULL if var == "full" else fc.FC_LADDER_PATH_REDUCED)
        assert fc.fc_message_block_weight_floats(cd, ld) == n
        assert fc.fc_message_block_workspace_bytes(cd, ld) > 0
    bad = fc.ladder_desc(216, 32, 3, 3, 1, 3, fc.FC_LADDER_PATH_REDUCED)   # ladder l_out must be 0
    assert fc.fc_message_block_weight_floats(fc.conv_desc(216, 1000, 32, 0, 3, 3, 5.0), bad) == 0


def test_vjp_vjp_w_argument_checks():
    """The explicit-weight VJP-of-VJP rejects an uninstantiated rank set and
    a call with no output on the host (no GPU call)."""
    import ctypes
    L = fc.lib()
    g = fc.Graph()
    d = fc.conv_desc(4, 8, 8, 5, 5, 5, 5.0)
    st = L.fc_edge_conv_vjp_vjp_w(ctypes.byref(d), ctypes.byref(g), *([None] * 12), None, 0, None)
    assert st == fc.FC_ERR_UNSUPPORTED
    d = fc.conv_desc(4, 8, 8, 2, 2, 2, 5.0)
    st = L.fc_edge_conv_vjp_vjp_w(ctypes.byref(d), ctypes.byref(g), *([None] * 12), None, 0, None)
    assert st == fc.FC_ERR_INVALID_ARGUMENT
    assert b"no output requested" in L.fc_last_error_message()


def test_vjp_vjp_instantiation_limits():
    """The fused-weight VJP-of-VJP covers rank 5 (its passes compiled as
    separate units); the explicit-weight one stops at rank 4 and says so
    before any launch."""
    import ctypes
    L = fc.lib()
    assert L.fc_edge_conv_workspace_bytes(ctypes.byref(fc.conv_desc(10, 20, 16, 5, 5, 5, 5.0)), 2) > 0
    d = fc.conv_desc(10, 20, 16, 5, 5, 5, 5.0)
    g = fc.Graph()
    st = L.fc_edge_conv_vjp_vjp_w(ctypes.byref(d), ctypes.byref(g), None, None, None, None, None, None, None, None,
                                  None, None, None, None, None, 0, None)
    assert st == fc.FC_ERR_UNSUPPORTED
    assert b"not instantiated" in L.fc_last_error_message()


def test_mlp_workspace_layouts():
    """Radial-network workspaces (host-side sizes only): the fused forward
    and force VJP hold per-edge hidden rows (512 bytes per edge); the
    materialised layouts hold w [E][P][C] (and w_bar); the VJP with the
    network's weight gradient (op 1) is materialised and covers op 2; other
    ops are refused (0 bytes).  Defaults: the forward fused at rank 2 and
    for the scalar-sender (0, 3, 3), materialised at (3, 3, 3); the VJP
    materialised unless FC_CONV_MLP_FUSE."""
    N, E, C = 1000, 64000, 128
    dflt = fc.conv_desc(N, E, C, 2, 2, 2, 5.0)
    fused = fc.conv_desc(N, E, C, 2, 2, 2, 5.0, flags=fc.FC_CONV_MLP_FUSE)
    mat = fc.conv_desc(N, E, C, 2, 2, 2, 5.0, flags=fc.FC_CONV_MLP_MATERIALIZE)
    P = fc.fc_conv_layout(fused)[0]
    f0, f1, f2 = (fc.fc_edge_conv_mlp_workspace_bytes(fused, op) for op in (0, 1, 2))
    m0, m1, m2 = (fc.fc_edge_conv_mlp_workspace_bytes(mat, op) for op in (0, 1, 2))
    d0, d2 = fc.fc_edge_conv_mlp_workspace_bytes(dflt, 0), fc.fc_edge_conv_mlp_workspace_bytes(dflt, 2)
    assert f0 == (E * 512 + 255) // 256 * 256 and d0 == f0
    assert m0 >= E * P * C * 4 and m2 >= 2 * E * P * C * 4 and d2 == m2
    assert f1 == m1 and f2 < f1 and f2 < m2
    assert fc.fc_edge_conv_mlp_workspace_bytes(fused, 3) == 0
    blk = dict(n_nodes=N, n_edges=E, channels=C, l_in=0, l_edge=3, l_out=3, r_cut=5.0)
    P4 = 4
    assert fc.fc_edge_conv_mlp_workspace_bytes(fc.conv_desc(**blk), 2) >= 2 * E * P4 * C * 4
    assert fc.fc_edge_conv_mlp_workspace_bytes(fc.conv_desc(**blk, flags=fc.FC_CONV_MLP_FUSE), 2) < E * P4 * C * 4
    assert fc.fc_edge_conv_mlp_workspace_bytes(fc.conv_desc(**blk), 0) < E * P4 * C * 4   # forward fused
    r3 = fc.conv_desc(N, E, C, 3, 3, 3, 5.0)
    assert fc.fc_edge_conv_mlp_workspace_bytes(r3, 0) >= E * fc.fc_conv_layout(r3)[0] * C * 4   # materialised
    # ranks above the fused set, and every-parity or summed outputs, are materialised
    for d in (fc.conv_desc(N, E, C, 4, 4, 4, 5.0), fc.conv_desc(N, E, C, 2, 2, 2, 5.0, flags=fc.FC_CONV_SUM_PATHS)):
        P2 = fc.fc_conv_layout(d)[0]
        assert fc.fc_edge_conv_mlp_workspace_bytes(d, 0) >= E * P2 * C * 4
