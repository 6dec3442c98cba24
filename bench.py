"""Benchmark of the FlashCart edge convolution on one MI355X.

One step = forward (Eq. 1) + VJP (feature and position gradients) of the
edge convolution on the 1024-node microbenchmark: positions uniform in a
20 A cube, 128 neighbours per node (E = 131072), 128 channels, ranks <= 2
(11 paths), Bessel-8 radial weights with r_c = 5 A; synthetic, seeded inputs
resident in HBM before timing starts.

Prints one JSON line: edge-channels/s = E*C / (t_fwd + t_vjp); the roofline
of the dominant kernel (the VJP): algorithmic flops per launch (exact
coupling-table counts) / its mean duration (HIP events on the launch stream)
against the FP32 vector ceiling, with the HBM figures beside it (algorithmic
gather bytes, compulsory bytes, and the counter-measured DRAM bytes when the
committed counters match the current kernel sources); and the oracle timed
on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F32_PEAK_TFS = 157.3
# FP32 vector ceilings: 256 CUs x 4 SIMDs, a wave64 VALU instruction takes 4
# cycles on its SIMD (16 lanes per cycle), 2.4 GHz.  Unpacked FMA:
# 256 * 4 * 16 * 2 flop * 2.4e9 = 78.6 TFLOP/s, i.e. 6.14e11 wave64
# instructions/s; packed FP32 (two lanes' FMAs per instruction) doubles this
# to 157.3, but this library is built with packed FP32 disabled.
VALU_F32_PEAK_TFS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
VALU_ISSUE_PER_S = 256 * 4 * 2.4e9 / 4
VALU_F32_PACKED_PEAK_TFS = 157.3
N_NODES, K_NBR, BOX, CHANNELS, LMAX, R_CUT, SEED = 1024, 128, 20.0, 128, 2, 5.0, 1
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_conv_vjp_sender_micro.json")


def measured_traffic():
    """HBM bytes per launch of the VJP sender kernel from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE runs, if the kernel is unchanged since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except OSError:
        return None
    from cartesian_tensor_product_amd.pmc import edge_kernel_source_sha
    if t.get("kernel_source_sha") != edge_kernel_source_sha():
        return None
    return t["bytes_per_launch"]


def timed(fn, iters=10, warmup=2):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(iters):
        fn()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def message_blocks(dev, cases=((8, "path_reduced"), (8, "full"), (5, "path_reduced"), (8, "path_reduced", "fused"))):
    """One full message-passing block (radial network, rank-wise map,
    residuals, RMS norms, SiLU gates, ladder of order 5, readout) for energy
    and forces on diamond cells of ncell^3 conventional cells, random weights;
    the radial network's output layer as the library chooses (materialised
    for this convolution), or (a third case entry) "fused" / "materialized"."""
    import torch

    from cartesian_tensor_product_amd import flashcart as fc
    from cartesian_tensor_product_amd import inputs as inp
    out = {}
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    en = torch.zeros(1, dtype=torch.float64, device=dev)
    variants = {"path_reduced": fc.FC_LADDER_PATH_REDUCED, "full": fc.FC_LADDER_FULL}
    for case in cases:
        ncell, vname, radial = (*case, "default")[:3]
        var = variants[vname]
        dm = inp.diamond_inputs(channels=CHANNELS, r_cut=5.0, rattle=0.05, ncell=ncell, n_paths=4)
        Nm, Em = dm["pos"].shape[0], len(dm["sender"])
        flags = {"default": 0, "fused": fc.FC_CONV_MLP_FUSE, "materialized": fc.FC_CONV_MLP_MATERIALIZE}[radial]
        cdm = fc.conv_desc(Nm, Em, CHANNELS, 0, 3, 3, 5.0, flags=flags)
        ldm = fc.ladder_desc(Nm, CHANNELS, 3, 3, 0, 5, var)
        C2 = CHANNELS
        entries = [("mlp", (4, C2), "mlp", 1), ("Mpre", (C2, C2), "normal", C2), ("M", (4, C2, C2), "normal", C2),
                   ("R0", (C2, C2), "normal", C2),
                   ("gamma1", (4, C2), "one_plus", 1), ("O", (4, C2, C2), "normal", C2)]
        entries += [(f"ladder{i}", (r_, c_), "normal" if k_ == 0 else "one_plus", c_)
                    for i, (_, r_, c_, k_) in enumerate(fc.ladder_weight_blocks(ldm))]
        entries += [("R2", (C2, C2), "normal", C2), ("gamma2", (1, C2), "one_plus", 1),
                    ("Wr1", (C2, 64), "normal", C2), ("Wr2", (64, 64), "normal", 64), ("wr3", (64,), "normal", 64)]
        wdict = inp.block_weights(8, entries)
        flat = t(np.concatenate([wdict[e[0]].ravel() for e in entries]))
        assert flat.numel() == fc.fc_message_block_weight_floats(cdm, ldm)
        gm = fc.DeviceGraph(dm["rowptr"], dm["sender"], Nm, device=dev)
        wsm = fc.workspace(fc.fc_message_block_workspace_bytes(cdm, ldm), dev)
        Fm = torch.empty((Nm, 3), device=dev)
        am = (cdm, gm, t(dm["pos"]), t(dm["shift"]), t(dm["x"]), ldm, flat, 1.0 / np.sqrt(Em / Nm), 1e-5)
        msm = timed(lambda: fc.fc_message_block_energy_forces(*am, en, None, Fm, wsm), iters=5)
        mse = timed(lambda: fc.fc_message_block_energy_forces(*am, en, None, None, wsm), iters=5)
        out[f"message_block_diamond_{Nm}_atoms_{vname}_order5" + ("" if radial == "default" else f"_radial_{radial}")] = {
            "energy_forces_ms": msm, "us_per_atom": msm * 1e3 / Nm, "energy_only_ms": mse, "edges": Em,
            "workspace_bytes": fc.fc_message_block_workspace_bytes(cdm, ldm)}
        del wsm, gm, flat
    return out


def radial_mlp_workload(dev):
    """The pages' radial network (Chebyshev + envelope + bias-free SiLU MLP)
    weighting the rank-2 micro convolution: its output layer fused into the
    convolution's lanes against w stored by an MFMA GEMM and streamed."""
    import torch

    from cartesian_tensor_product_amd import flashcart as fc
    from cartesian_tensor_product_amd import inputs
    out = {}
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    desc = fc.conv_desc(N_NODES, N_NODES * K_NBR, CHANNELS, 2, 2, 2, R_CUT)
    P, n_in, n_out = fc.fc_conv_layout(desc)
    d = inputs.edge_conv_inputs(1, N_NODES, K_NBR, BOX, CHANNELS, n_in, P, n_out)
    mlp = t(inputs.radial_mlp_weights(np.random.default_rng(51), P, CHANNELS))
    graph = fc.DeviceGraph(d["rowptr"], d["sender"], N_NODES, device=dev)
    pos, x, g = t(d["pos"]), t(d["x"]), t(d["g"])
    E = N_NODES * K_NBR
    w = torch.empty((E, P, CHANNELS), device=dev)
    z = torch.empty((N_NODES, n_out, CHANNELS), device=dev)
    xb, pb, mb = torch.empty_like(x), torch.empty((N_NODES, 3), device=dev), torch.empty_like(mlp)
    from cartesian_tensor_product_amd.opcount import conv_fma_per_edge_channel
    ops64 = conv_fma_per_edge_channel(2, 2, 2, n_basis=64)
    r = {"w_bytes": E * P * CHANNELS * 4, "fused_fma_per_edge_channel": ops64}
    for mode, flags in (("fused", fc.FC_CONV_MLP_FUSE), ("materialized", fc.FC_CONV_MLP_MATERIALIZE)):
        dm = fc.conv_desc(N_NODES, E, CHANNELS, 2, 2, 2, R_CUT, flags=flags)
        ws0 = fc.workspace(fc.fc_edge_conv_mlp_workspace_bytes(dm, 0), dev)
        ws2 = fc.workspace(fc.fc_edge_conv_mlp_workspace_bytes(dm, 2), dev)
        fms = timed(lambda: fc.fc_edge_conv_mlp_fwd(dm, graph, pos, None, x, mlp, z, ws0))
        vms = timed(lambda: fc.fc_edge_conv_mlp_vjp(dm, graph, pos, None, x, mlp, g, xb, pb, None, ws2))
        r[mode] = {"fwd_ms": fms, "vjp_x_pos_ms": vms,
                   "fwd_plus_vjp_edge_channels_per_s": E * CHANNELS / ((fms + vms) * 1e-3),
                   # fused: FMAs per edge-channel with the 64 hidden units as the basis
                   "fwd_alu_frac": (2.0 * ops64["fwd"] * E * CHANNELS / (fms * 1e-3) / 1e12 / VALU_F32_PEAK_TFS
                                    if mode == "fused" else None),
                   "vjp_alu_frac": (2.0 * ops64["vjp"] * E * CHANNELS / (vms * 1e-3) / 1e12 / VALU_F32_PEAK_TFS
                                    if mode == "fused" else None),
                   "workspace_bytes_fwd": fc.fc_edge_conv_mlp_workspace_bytes(dm, 0),
                   "workspace_bytes_vjp": fc.fc_edge_conv_mlp_workspace_bytes(dm, 2)}
        del ws0, ws2
    ws1 = fc.workspace(fc.fc_edge_conv_mlp_workspace_bytes(desc, 1), dev)
    rms = timed(lambda: fc.fc_radial_mlp(desc, graph, pos, None, mlp, w, ws1))
    r["radial_mlp_w_only_ms"] = rms
    r["output_layer_tflops_lower_bound"] = 2.0 * E * 64 * P * CHANNELS / (rms * 1e-3) / 1e12
    r["vjp_with_mlp_grad_ms"] = timed(lambda: fc.fc_edge_conv_mlp_vjp(desc, graph, pos, None, x, mlp, g, xb, pb, mb,
                                                                      ws1))
    r["fused_speedup_fwd_plus_vjp"] = ((r["materialized"]["fwd_ms"] + r["materialized"]["vjp_x_pos_ms"]) /
                                      (r["fused"]["fwd_ms"] + r["fused"]["vjp_x_pos_ms"]))
    r["default"] = "forward fused, VJP materialised (at these ranks)"
    out["conv_radial_mlp_rank2_1024n_128c_128nbr"] = r
    del w, z, xb, pb, mb, ws1, mlp
    return out


def extras(dev, only_ladder=False, conv_ranks=(3, 4), only_conv=False):
    """Secondary workloads (reported beside the headline, not part of it)."""
    import torch

    from cartesian_tensor_product_amd import flashcart as fc
    from cartesian_tensor_product_amd import inputs
    out = {}
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    # high-rank microbenchmark: fwd, VJP, VJP-of-VJP (position cotangent)
    for l in (() if only_ladder else conv_ranks):
        desc = fc.conv_desc(N_NODES, N_NODES * K_NBR, CHANNELS, l, l, l, R_CUT)
        P, n_in, n_out = fc.fc_conv_layout(desc)
        d = inputs.edge_conv_inputs(2, N_NODES, K_NBR, BOX, CHANNELS, n_in, P, n_out, with_vpos=True)
        graph = fc.DeviceGraph(d["rowptr"], d["sender"], N_NODES, device=dev)
        pos, x, W, g, vp = t(d["pos"]), t(d["x"]), t(d["W"]), t(d["g"]), t(d["v_pos"])
        z = torch.empty((N_NODES, n_out, CHANNELS), device=dev)
        xb, pb = torch.empty_like(x), torch.empty((N_NODES, 3), device=dev)
        gh, xh, ph = torch.empty_like(z), torch.empty_like(x), torch.empty_like(pb)
        ws = fc.workspace(max(fc.fc_edge_conv_workspace_bytes(desc, 1), fc.fc_edge_conv_workspace_bytes(desc, 2)), dev)
        E = N_NODES * K_NBR
        Wb = torch.empty_like(W)
        r = {"fwd_ms": timed(lambda: fc.fc_edge_conv_fwd(desc, graph, pos, None, x, W, z)),
             "vjp_ms": timed(lambda: fc.fc_edge_conv_vjp(desc, graph, pos, None, x, W, g, xb, pb, None, ws)),
             "radial_w_grad_ms": timed(lambda: fc.fc_edge_conv_vjp(desc, graph, pos, None, x, W, g, None, None, Wb,
                                                                   ws)),
             "vjp_vjp_ms": timed(lambda: fc.fc_edge_conv_vjp_vjp(desc, graph, pos, None, x, W, g, None, vp, None, gh, xh,
                                                                 ph, None, ws), iters=5),
             "radial_w_hat_ms": timed(lambda: fc.fc_edge_conv_vjp_vjp(desc, graph, pos, None, x, W, g, None, vp,
                                                                      None, None, None, None, Wb, ws), iters=5)}
        r["fwd_plus_vjp_edge_channels_per_s"] = E * CHANNELS / ((r["fwd_ms"] + r["vjp_ms"]) * 1e-3)
        out[f"conv_rank{l}_1024n_128c_128nbr"] = r
        del z, xb, pb, gh, xh, ph, ws, Wb
    # every triangle-allowed path (odd J through the Levi-Civita reading), the
    # literal path sets of the microbenchmark configurations: ranks <= 2
    # (15 paths), <= 3 (34), <= 4 (65)
    for l in (() if only_ladder else ((2, 3, 4) if not only_conv else ())):
        desc = fc.conv_desc(N_NODES, N_NODES * K_NBR, CHANNELS, l, l, l, R_CUT, flags=fc.FC_CONV_ALL_PARITIES)
        P, n_in, n_out = fc.fc_conv_layout(desc)
        d = inputs.edge_conv_inputs(1 if l == 2 else 2, N_NODES, K_NBR, BOX, CHANNELS, n_in, P, n_out,
                                    with_vpos=True)
        graph = fc.DeviceGraph(d["rowptr"], d["sender"], N_NODES, device=dev)
        pos, x, W, g, vp = t(d["pos"]), t(d["x"]), t(d["W"]), t(d["g"]), t(d["v_pos"])
        z = torch.empty((N_NODES, n_out, CHANNELS), device=dev)
        xb, pb = torch.empty_like(x), torch.empty((N_NODES, 3), device=dev)
        ws = fc.workspace(fc.fc_edge_conv_workspace_bytes(desc, 2), dev)
        E = N_NODES * K_NBR
        r = {"paths": P, "fwd_ms": timed(lambda: fc.fc_edge_conv_fwd(desc, graph, pos, None, x, W, z)),
             "vjp_ms": timed(lambda: fc.fc_edge_conv_vjp(desc, graph, pos, None, x, W, g, xb, pb, None, ws))}
        gh, xh, ph = torch.empty_like(z), torch.empty_like(x), torch.empty_like(pb)
        r["vjp_vjp_ms"] = timed(lambda: fc.fc_edge_conv_vjp_vjp(desc, graph, pos, None, x, W, g, None, vp, None, gh, xh,
                                                                ph, None, ws), iters=5)
        del gh, xh, ph
        r["fwd_plus_vjp_edge_channels_per_s"] = E * CHANNELS / ((r["fwd_ms"] + r["vjp_ms"]) * 1e-3)
        out[f"conv_all_parities_rank{l}_1024n_128c_128nbr"] = r
        del z, xb, pb, ws
    # path-summed outputs (one block per output rank): the micro workload at
    # ranks 2, 3, 4; z and g shrink from sum_L (2L+1) P_L rows to (l+1)^2
    for l in (() if only_ladder else ((2, 3, 4) if not only_conv else ())):
        desc = fc.conv_desc(N_NODES, N_NODES * K_NBR, CHANNELS, l, l, l, R_CUT, flags=fc.FC_CONV_SUM_PATHS)
        P, n_in, n_out = fc.fc_conv_layout(desc)
        d = inputs.edge_conv_inputs(1 if l == 2 else 2, N_NODES, K_NBR, BOX, CHANNELS, n_in, P, n_out,
                                    with_vpos=True)
        graph = fc.DeviceGraph(d["rowptr"], d["sender"], N_NODES, device=dev)
        pos, x, W, g, vp = t(d["pos"]), t(d["x"]), t(d["W"]), t(d["g"]), t(d["v_pos"])
        z = torch.empty((N_NODES, n_out, CHANNELS), device=dev)
        xb, pb = torch.empty_like(x), torch.empty((N_NODES, 3), device=dev)
        ws = fc.workspace(fc.fc_edge_conv_workspace_bytes(desc, 2), dev)
        E = N_NODES * K_NBR
        r = {"out_rows": n_out, "fwd_ms": timed(lambda: fc.fc_edge_conv_fwd(desc, graph, pos, None, x, W, z)),
             "vjp_ms": timed(lambda: fc.fc_edge_conv_vjp(desc, graph, pos, None, x, W, g, xb, pb, None, ws))}
        gh, xh, ph = torch.empty_like(z), torch.empty_like(x), torch.empty_like(pb)
        r["vjp_vjp_ms"] = timed(lambda: fc.fc_edge_conv_vjp_vjp(desc, graph, pos, None, x, W, g, None, vp, None,
                                                                gh, xh, ph, None, ws), iters=5)
        del gh, xh, ph
        r["fwd_plus_vjp_edge_channels_per_s"] = E * CHANNELS / ((r["fwd_ms"] + r["vjp_ms"]) * 1e-3)
        out[f"conv_summed_rank{l}_1024n_128c_128nbr"] = r
        del z, xb, pb, ws
    if not only_ladder and not only_conv:
        out.update(radial_mlp_workload(dev))
    # equivariant RMS normalisation of the ladder's node features (4096
    # nodes, 128 channels, ranks <= 3): forward, and VJP with both gradients
    if not only_conv:
        nd = fc.norm_desc(4096, CHANNELS, 3, 1e-5)
        rng = np.random.default_rng(5)
        xn = t(inputs.normal(rng, (4096, 16, CHANNELS)))
        gam = t(inputs.f32(1.0 + 0.1 * rng.standard_normal((4, CHANNELS))))
        gy = t(inputs.normal(rng, (4096, 16, CHANNELS)))
        yn, isn, xnb, gamb = torch.empty_like(xn), torch.empty(4096, device=dev), torch.empty_like(xn), torch.empty_like(gam)
        wsn = fc.workspace(fc.fc_rms_norm_workspace_bytes(nd), dev)
        fms = timed(lambda: fc.fc_rms_norm_fwd(nd, xn, gam, yn, isn))
        vms = timed(lambda: fc.fc_rms_norm_vjp(nd, xn, gam, isn, gy, xnb, gamb, wsn))
        nb = 4096 * 16 * CHANNELS * 4
        out["rms_norm_4096n_128c_rank3"] = {"fwd_ms": fms, "vjp_ms": vms,
                                            "fwd_GBs_compulsory": 2 * nb / (fms * 1e-3) / 1e9,
                                            "vjp_GBs_compulsory": 3 * nb / (vms * 1e-3) / 1e9}
        del xn, gy, yn, xnb, wsn
    # node-local ladder, 4096 nodes, 128 channels, ranks <= 3, order 4, both variants
    for name, var in (() if only_conv else (("full", fc.FC_LADDER_FULL), ("path_reduced", fc.FC_LADDER_PATH_REDUCED))):
        ld = fc.ladder_desc(4096, CHANNELS, 3, 3, 3, 4, var)
        blocks = fc.ladder_weight_blocks(ld)
        shapes = [((r, c), "normal" if kind == 0 else "one_plus", c) for (_, r, c, kind) in blocks]
        rng, A, ws = inputs.ladder_inputs(3, 4096, CHANNELS, 16, shapes)
        gz = inputs.ladder_cotangent(rng, 4096, 16, CHANNELS)
        dA, dW, dg = t(A), t(np.concatenate([w.ravel() for w in ws])), t(gz)
        nw, ns = fc.fc_ladder_layout(ld)
        saved = torch.empty(ns, device=dev)
        z = torch.empty((4096, 16, CHANNELS), device=dev)
        Ab, Wb = torch.empty_like(dA), torch.empty_like(dW)
        wsf = fc.workspace(fc.fc_ladder_workspace_bytes(ld, 0), dev)
        wsb = fc.workspace(fc.fc_ladder_workspace_bytes(ld, 1), dev)
        r = {"fwd_ms": timed(lambda: fc.fc_node_ladder_fwd(ld, dA, dW, z, saved, wsf)),
             "vjp_ms": timed(lambda: fc.fc_node_ladder_vjp(ld, dA, dW, saved, dg, Ab, Wb, wsb))}
        r["node_channels_per_s_fwd"] = 4096 * CHANNELS / (r["fwd_ms"] * 1e-3)
        # VJP-of-VJP with the cotangent on A_grad only (zero weight-gradient
        # cotangent, as the pages time it); its workspace is the extra memory
        fc.fc_node_ladder_fwd(ld, dA, dW, z, saved, wsf)
        vA = t(inputs.normal(np.random.default_rng(6), A.shape))
        gh, Ah, Wh = torch.empty_like(z), torch.empty_like(dA), torch.empty_like(dW)
        wsv = fc.workspace(fc.fc_ladder_workspace_bytes(ld, 2), dev)
        r["vjp_vjp_ms"] = timed(lambda: fc.fc_node_ladder_vjp_vjp(ld, dA, dW, saved, dg, vA, None, gh, Ah, Wh,
                                                                  wsv), iters=5)
        r["vjp_vjp_workspace_bytes"] = fc.fc_ladder_workspace_bytes(ld, 2)
        del vA, gh, Ah, Wh, wsv
        out[f"ladder_{name}_4096n_128c_rank3_order4"] = r
        del saved, z, Ab, Wb, wsf, wsb
    if only_conv:
        return out
    out["ladder_full_4096n_128c_rank3_order4"]["mixing_gemm_gflop_fwd"] = ladder_gemm_gflop(4096, CHANNELS, 3, 4)
    lf = out["ladder_full_4096n_128c_rank3_order4"]
    lf["mixing_gemm_tflops_fwd_lower_bound"] = lf["mixing_gemm_gflop_fwd"] / lf["fwd_ms"]
    if only_ladder:
        return out
    # 1000-atom diamond block: energy and forces
    from cartesian_tensor_product_amd import inputs as inp
    cd_l = fc.ladder_desc(1000, CHANNELS, 3, 3, 0, 5, fc.FC_LADDER_PATH_REDUCED)
    blocks = fc.ladder_weight_blocks(cd_l)
    shapes = [((r_, c_), "normal" if k_ == 0 else "one_plus", c_) for (_, r_, c_, k_) in blocks]
    dd = inp.diamond_inputs(channels=CHANNELS, r_cut=5.0, rattle=0.05, n_paths=4, ladder_weight_shapes=shapes)
    Nd, Ed = dd["pos"].shape[0], len(dd["sender"])
    cd = fc.conv_desc(Nd, Ed, CHANNELS, 0, 3, 3, 5.0)
    graph = fc.DeviceGraph(dd["rowptr"], dd["sender"], Nd, device=dev)
    lw = t(np.concatenate([w.ravel() for w in dd["ladder_weights"]]))
    en = torch.zeros(1, dtype=torch.float64, device=dev)
    F = torch.empty((Nd, 3), device=dev)
    wsd = fc.workspace(fc.fc_block_workspace_bytes(cd, cd_l), dev)
    args = (cd, graph, t(dd["pos"]), t(dd["shift"]), t(dd["x"]), t(dd["W"]), cd_l, lw, 1.0 / np.sqrt(Ed / Nd))
    ms = timed(lambda: fc.fc_block_energy_forces(*args, en, None, F, wsd))
    out["diamond_1000_atoms_energy_forces"] = {"ms": ms, "us_per_atom": ms * 1e3 / Nd, "edges": Ed}
    del wsd
    out.update(message_blocks(dev))
    return out


def ladder_gemm_gflop(N, C, l, order):
    """Flops of the full ladder's mixing GEMMs in one forward: W1 on every
    rank, then per step sum_L 2 N (2L+1) (P_L C) C with P_L the admissible
    paths (l1 <= l, l2 <= l) -> L."""
    def paths(L):
        return sum(1 for a in range(l + 1) for b in range(l + 1)
                   if abs(a - b) <= L <= a + b and (a + b + L) % 2 == 0)
    f = sum(2.0 * N * (2 * L + 1) * C * C for L in range(l + 1))
    f += (order - 1) * sum(2.0 * N * (2 * L + 1) * paths(L) * C * C for L in range(l + 1))
    return f / 1e9


def copy_bandwidth(mb=1024, iters=20):
    """Device-to-device copy rate (read + write bytes per second, GB/s) of a
    plain copy of mb MiB: the bandwidth a streaming kernel can reach here."""
    import torch
    src = torch.ones(mb * (1 << 20) // 4, device="cuda:0")
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src), iters)
    del src, dst
    return 2 * mb * (1 << 20) / (ms * 1e-3) / 1e9


def algorithmic_bytes(N, E, C, n_in, n_out, P):
    """Bytes each launch must move if every per-edge gather goes to memory.

    forward: gather x[v] (n_in C floats) per edge, write z once per node,
             sender id + sender position per edge, rowptr + receiver position
             per node, radial weights once.
    VJP:     gather g[u] (n_out C floats) per edge, read x[v] and write x_bar[v]
             once per node, per edge the edge id, receiver id, receiver
             position, and the edge position cotangent (written, then read by
             the receiver pass), positions/row pointers and pos_bar per node,
             radial weights once.
    """
    f = 4
    fwd = E * C * n_in * f + N * n_out * C * f + E * (4 + 12) + N * (8 + 12) + 8 * P * C * f
    vjp = (E * C * n_out * f + 2 * N * n_in * C * f + E * (4 + 4 + 12 + 12 + 12) + N * (8 + 8 + 12 + 12 + 12)
           + 8 * P * C * f)
    return fwd, vjp


def compulsory_bytes(N, E, C, n_in, n_out, P, explicit=False):
    """Bytes no schedule can avoid: every array read or written once (x, z or
    g, x_bar, positions, graph, per-edge position cotangents), plus w and
    w_bar with explicit per-edge weights; gathers served from cache are not
    counted again."""
    f = 4
    graph = E * 4 + N * 4 * 2 + N * 12
    fwd = N * n_in * C * f + N * n_out * C * f + graph + (E * P * C * f if explicit else 8 * P * C * f)
    vjp = (N * n_out * C * f + 2 * N * n_in * C * f + graph * 2 + E * 12 * 2 + N * 12
           + (2 * E * P * C * f if explicit else 8 * P * C * f))
    return fwd, vjp


def grid(dev, steps):
    """The pages' microbenchmark grid (1024 nodes x {64, 128} neighbours x
    {64, 128, 256} channels x ranks 1-5): forward, VJP and VJP-of-VJP
    (position cotangent) with fused Bessel radial weights, and
    forward + VJP with explicit per-edge weights drawn on the device."""
    import torch

    from cartesian_tensor_product_amd import flashcart as fc
    from cartesian_tensor_product_amd import inputs
    rows = []
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    for k in (64, 128):
        rng, pos_h, rowptr, sender = inputs.random_cloud(SEED, N_NODES, k, BOX)
        graph = fc.DeviceGraph(rowptr, sender, N_NODES, device=dev)
        pos = t(pos_h)
        E = len(sender)
        for C in (64, 128, 256):
            for l in (1, 2, 3, 4, 5):
                desc = fc.conv_desc(N_NODES, E, C, l, l, l, R_CUT)
                P, n_in, n_out = fc.fc_conv_layout(desc)
                gen = torch.Generator(device=dev).manual_seed(1000 * k + 10 * C + l)
                rn = lambda shape, std=1.0: torch.randn(shape, device=dev, generator=gen) * std
                x, g = rn((N_NODES, n_in, C)), rn((N_NODES, n_out, C))
                W, vp = rn((8, P, C), 8 ** -0.5), rn((N_NODES, 3))
                z, xb, pb = torch.empty_like(g), torch.empty_like(x), torch.empty_like(pos)
                ws = fc.workspace(max(fc.fc_edge_conv_workspace_bytes(desc, 1),
                                      fc.fc_edge_conv_workspace_bytes(desc, 2)), dev)
                r = {"neighbours": k, "channels": C, "l_max": l, "paths": P,
                     "fwd_ms": timed(lambda: fc.fc_edge_conv_fwd(desc, graph, pos, None, x, W, z), steps),
                     "vjp_ms": timed(lambda: fc.fc_edge_conv_vjp(desc, graph, pos, None, x, W, g, xb, pb, None, ws),
                                     steps),
                     "vjp_vjp_ms": timed(lambda: fc.fc_edge_conv_vjp_vjp(desc, graph, pos, None, x, W, g, None, vp,
                                                                         None, z, xb, pb, None, ws), max(2, steps // 4))}
                w = rn((E, P, C))
                wb = torch.empty_like(w)
                r["explicit_fwd_ms"] = timed(lambda: fc.fc_edge_conv_fwd_w(desc, graph, pos, None, x, w, z), steps)
                r["explicit_vjp_ms"] = timed(
                    lambda: fc.fc_edge_conv_vjp_w(desc, graph, pos, None, x, w, g, xb, pb, wb, ws), steps)
                bf, bv = compulsory_bytes(N_NODES, E, C, n_in, n_out, P, explicit=True)
                r["explicit_fwd_plus_vjp_frac_hbm_compulsory"] = (
                    (bf + bv) / ((r["explicit_fwd_ms"] + r["explicit_vjp_ms"]) * 1e-3) / 1e9 / HBM_PEAK_GBS)
                r["fwd_plus_vjp_edge_channels_per_s"] = E * C / ((r["fwd_ms"] + r["vjp_ms"]) * 1e-3)
                rows.append(r)
                print(json.dumps(r), file=sys.stderr, flush=True)
                del x, g, W, vp, z, xb, pb, ws, w, wb
    return rows


# --------------------------------------------------------- the CPU oracle --
# Worker processes (spawned, so they touch no GPU state) regenerate the
# seeded inputs once in their initializer, outside the timed region, and
# evaluate the oracle on a share of the workload with one BLAS thread each.

_W = {}


def _conv_worker_init(ranks, r_cut):
    from threadpoolctl import threadpool_limits

    from cartesian_tensor_product_amd import inputs
    from oracle import conv
    _W["limit"] = threadpool_limits(limits=1)
    spec = conv.ConvSpec(*ranks, r_cut)
    d = inputs.edge_conv_inputs(SEED, N_NODES, K_NBR, BOX, CHANNELS, spec.n_in, spec.n_paths, spec.n_out)
    f = lambda a: a.astype(np.float64)
    _W["conv"] = (spec, f(d["pos"]), d["rowptr"], d["sender"], f(d["x"]), f(d["W"]), f(d["g"]))


def _conv_worker(edge_range):
    from oracle import conv
    spec, pos, rowptr, sender, x, W, g = _W["conv"]
    edges = np.arange(*edge_range)
    z = conv.edge_conv_fwd(spec, pos, rowptr, sender, x, W, edges=edges)
    xb, pb, _ = conv.edge_conv_vjp(spec, pos, rowptr, sender, x, W, g, edges=edges)
    return float(z.sum() + xb.sum() + pb.sum())


def _ladder_worker_init(n_nodes):
    from threadpoolctl import threadpool_limits

    from cartesian_tensor_product_amd import inputs
    from oracle import ladder
    _W["limit"] = threadpool_limits(limits=1)
    for variant in ("reduced", "full"):
        spec = ladder.LadderSpec(3, 3, 3, 4, variant, CHANNELS)
        shapes = [(sh[1], sh[2], sh[3]) for sh in spec.weight_shapes()]
        rng, A, ws = inputs.ladder_inputs(3, n_nodes, CHANNELS, 16, shapes)
        gz = inputs.ladder_cotangent(rng, n_nodes, 16, CHANNELS)
        _W[variant] = (spec, A.astype(np.float64), [w.astype(np.float64) for w in ws], gz.astype(np.float64))


def _ladder_worker(task):
    from oracle import ladder
    variant, lo, hi = task
    spec, A, ws, gz = _W[variant]
    nodes = np.arange(lo, hi)
    z = ladder.ladder_fwd(spec, A, ws, nodes=nodes)
    Ab, _ = ladder.ladder_vjp(spec, A, ws, gz, nodes=nodes)
    return float(z.sum() + Ab.sum())


def host_cores():
    """Cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS
    where the environment sets the process's CPU share."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline():
    """The oracle (numpy fp64, probed bilinear maps) on the host cores, one
    worker process per core: the whole edge-conv workload (fwd + VJP of all
    131072 edges) and the 4096-node ladder (rank 3, order 4, fwd + VJP, both
    variants), wall-clock of the parallel map."""
    import multiprocessing as mp
    cores = host_cores()
    ctx = mp.get_context("spawn")
    out = {"unit": "edge-channels/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model()}
    E = N_NODES * K_NBR
    per = (N_NODES + 4 * cores - 1) // (4 * cores)          # receivers per task
    tasks = [(r * K_NBR, min(N_NODES, r + per) * K_NBR) for r in range(0, N_NODES, per)]
    with ctx.Pool(cores, initializer=_conv_worker_init, initargs=((LMAX, LMAX, LMAX), R_CUT)) as pool:
        pool.map(_conv_worker, [(0, 1)] * cores, chunksize=1)          # workers initialised
        t0 = time.perf_counter()
        pool.map(_conv_worker, tasks, chunksize=1)
        dt = time.perf_counter() - t0
    out["value"] = E * CHANNELS / dt
    out["sample"] = (f"the whole workload: fwd + VJP (x_grad, pos_grad) of all {E} edges x {CHANNELS} channels, "
                     f"{len(tasks)} receiver-range tasks over {cores} processes, {dt:.1f} s")
    n_lad = min(4096, 512 * cores)
    with ctx.Pool(cores, initializer=_ladder_worker_init, initargs=(n_lad,)) as pool:
        pool.map(_ladder_worker, [("reduced", 0, 1)] * cores, chunksize=1)
        lad = {}
        for variant in ("reduced", "full"):
            t0 = time.perf_counter()
            pool.map(_ladder_worker, [(variant, lo, min(n_lad, lo + 128)) for lo in range(0, n_lad, 128)],
                     chunksize=1)
            dt = time.perf_counter() - t0
            lad[variant] = {"node_channels_per_s_fwd_plus_vjp": n_lad * CHANNELS / dt, "nodes": n_lad,
                            "seconds": dt}
    out["ladder_4096n_128c_rank3_order4"] = {"path_reduced": lad["reduced"], "full": lad["full"],
                                            "unit": "node-channels/s (fwd + VJP)"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--ladder-only", action="store_true",
                    help="only run the 4096-node ladder workloads (for counter runs) and print their timings")
    ap.add_argument("--conv-rank", type=int, default=0, metavar="L",
                    help="only run the 1024-node edge-conv workload at ranks <= L (3 or 4; for counter runs)")
    ap.add_argument("--mlp-only", action="store_true",
                    help="only run the radial-network convolution workload (fused and materialised)")
    ap.add_argument("--message-block-only", action="store_true",
                    help="only time the path-reduced message block on the 4096-atom diamond cell")
    ap.add_argument("--grid", action="store_true",
                    help="only run the pages' microbenchmark grid (ranks 1-5) and print it as one JSON line")
    ap.add_argument("--copy-only", type=int, default=0, metavar="MB",
                    help="only run 5 device-to-device copies of MB megabytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_only:
        src = torch.ones(args.copy_only * (1 << 20) // 4, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 4, "copies": 5}))
        return

    from cartesian_tensor_product_amd import flashcart as fc
    from cartesian_tensor_product_amd import inputs

    dev = torch.device("cuda:0")
    if args.ladder_only:
        print(json.dumps(extras(dev, only_ladder=True)), flush=True)
        return
    if args.grid:
        print(json.dumps({"grid": grid(dev, 10)}), flush=True)
        return
    if args.message_block_only:
        print(json.dumps(message_blocks(dev, ((8, "path_reduced"),))), flush=True)
        return
    if args.mlp_only:
        print(json.dumps(radial_mlp_workload(dev)), flush=True)
        return
    if args.conv_rank:
        print(json.dumps(extras(dev, conv_ranks=(args.conv_rank,), only_conv=True)), flush=True)
        return
    desc = fc.conv_desc(N_NODES, N_NODES * K_NBR, CHANNELS, LMAX, LMAX, LMAX, R_CUT)
    P, n_in, n_out = fc.fc_conv_layout(desc)
    d = inputs.edge_conv_inputs(SEED, N_NODES, K_NBR, BOX, CHANNELS, n_in, P, n_out)
    E = len(d["sender"])
    graph = fc.DeviceGraph(d["rowptr"], d["sender"], N_NODES, device=dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    pos, x, W, g = t(d["pos"]), t(d["x"]), t(d["W"]), t(d["g"])
    z = torch.empty((N_NODES, n_out, CHANNELS), device=dev)
    xb = torch.empty_like(x)
    pb = torch.empty((N_NODES, 3), device=dev)
    ws = fc.workspace(fc.fc_edge_conv_workspace_bytes(desc, 1), dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fc.fc_edge_conv_fwd(desc, graph, pos, None, x, W, z, stream)
        if ev is not None:
            ev[1].record(stream)
        fc.fc_edge_conv_vjp(desc, graph, pos, None, x, W, g, xb, pb, None, ws, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_fwd = np.array([e[0].elapsed_time(e[1]) for e in evs])
    t_vjp = np.array([e[1].elapsed_time(e[2]) for e in evs])
    ms_step = float(evs[0][0].elapsed_time(evs[-1][2]) / args.steps)

    b_fwd, b_vjp = algorithmic_bytes(N_NODES, E, CHANNELS, n_in, n_out, P)
    c_fwd, c_vjp = compulsory_bytes(N_NODES, E, CHANNELS, n_in, n_out, P)
    from cartesian_tensor_product_amd.opcount import conv_fma_per_edge_channel
    ops = conv_fma_per_edge_channel(LMAX, LMAX, LMAX)
    f_mean, v_mean = float(t_fwd.mean()), float(t_vjp.mean())
    value = E * CHANNELS / (ms_step * 1e-3)

    def ceilings(ms, fma, alg_bytes, comp_bytes, traffic):
        """Both ceilings of one launch: the FP32 vector one from the exact
        FMA count, and HBM from the gather model, the compulsory bytes and
        (if measured for these sources) the counter bytes."""
        sec = ms * 1e-3
        tf = 2.0 * fma * E * CHANNELS / sec / 1e12
        hbm = {"algorithmic_bytes_per_launch": alg_bytes, "gather_model_GBs": alg_bytes / sec / 1e9,
               "gather_model_frac": alg_bytes / sec / 1e9 / HBM_PEAK_GBS,
               "compulsory_bytes_per_launch": comp_bytes, "compulsory_GBs": comp_bytes / sec / 1e9,
               "counter_bytes_per_launch": traffic,
               "counter_GBs": None if traffic is None else traffic / sec / 1e9,
               "counter_frac": None if traffic is None else traffic / sec / 1e9 / HBM_PEAK_GBS}
        alu = {"fma_per_edge_channel": fma, "algorithmic_flops_per_launch": 2.0 * fma * E * CHANNELS,
               "TFLOPs": tf, "frac": tf / VALU_F32_PEAK_TFS,
               "wave_instructions_per_s_lower_bound": fma * E * CHANNELS / 64 / sec,
               "frac_of_packed_fp32_peak": tf / VALU_F32_PACKED_PEAK_TFS}
        # the nearer ceiling: DRAM is judged by the bytes that reach it (the
        # counters, else the compulsory bytes), not by cache-served gathers
        dram_frac = hbm["counter_frac"] if traffic is not None else comp_bytes / sec / 1e9 / HBM_PEAK_GBS
        return hbm, alu, ("alu" if alu["frac"] >= dram_frac else "hbm")

    traffic = measured_traffic()
    hbm_v, alu_v, bound_v = ceilings(v_mean, ops["vjp"], b_vjp, c_vjp, traffic)
    hbm_f, alu_f, bound_f = ceilings(f_mean, ops["fwd"], b_fwd, c_fwd, None)
    dom = "fc_edge_conv_vjp (conv_vjp_sender_kernel<2,2,2> + conv_vjp_combine_kernel)"
    if bound_v == "alu":
        roof = {"bound": "alu", "kernel": dom, "achieved": alu_v["TFLOPs"], "peak": VALU_F32_PEAK_TFS,
                "unit": "TFLOP/s", "frac": alu_v["frac"], "traffic": traffic,
                "algorithmic_flops_per_launch": alu_v["algorithmic_flops_per_launch"],
                "peak_note": "FP32 FMA without packed instructions (built with packed FP32 off); "
                             f"packed peak {VALU_F32_PACKED_PEAK_TFS}", "hbm": hbm_v}
    else:
        roof = {"bound": "hbm", "kernel": dom, "achieved": hbm_v["gather_model_GBs"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": hbm_v["gather_model_frac"], "traffic": traffic,
                "algorithmic_bytes_per_launch": b_vjp, "alu": alu_v}

    out = {
        "metric": "edge-conv fwd+VJP edge-channels/s (1024n,128c,128nbr); % HBM roofline",
        "value": value,
        "unit": "edge-channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "edge conv fwd+VJP, 1024 nodes, 128 neighbours (E=131072), 128 channels, "
                               "ranks<=2 (11 paths), Bessel-8 r_c=5 A, seed 1",
                   "nodes": N_NODES, "neighbours": K_NBR, "channels": CHANNELS, "l_max": LMAX,
                   "edges": E},
        "roofline": roof,
        "breakdown": {"fwd_ms": f_mean, "vjp_ms": v_mean,
                      "fwd_alu": alu_f, "fwd_hbm": hbm_f, "fwd_bound": bound_f,
                      "fwd_plus_vjp_gather_model_frac_hbm": (b_fwd + b_vjp) / ((f_mean + v_mean) * 1e-3) / 1e9
                      / HBM_PEAK_GBS,
                      "fwd_plus_vjp_frac_alu": 2.0 * (ops["fwd"] + ops["vjp"]) * E * CHANNELS
                      / ((f_mean + v_mean) * 1e-3) / 1e12 / VALU_F32_PEAK_TFS,
                      "wall_s": wall,
                      "fwd_ms_p10_p50_p90": [float(np.percentile(t_fwd, q)) for q in (10, 50, 90)],
                      "vjp_ms_p10_p50_p90": [float(np.percentile(t_vjp, q)) for q in (10, 50, 90)],
                      "vjp_workspace_bytes": fc.fc_edge_conv_workspace_bytes(desc, 1),
                      # the byte model of a receiver-sorted VJP with atomic x_bar
                      # updates (gather x and add into x_bar per edge-channel)
                      "vjp_bytes_receiver_atomics_model": 2 * E * CHANNELS * n_in * 4 + N_NODES * n_out * CHANNELS * 4},
    }
    cbw = copy_bandwidth()
    out["breakdown"]["copy_GBs_measured"] = cbw
    # the sender-sorted transpose of the graph (rebuilt whenever the
    # neighbour list changes; outside the timed step), rewritten in place
    # with the same values
    out["breakdown"]["graph_transpose_ms"] = timed(
        lambda: fc.fc_graph_transpose(N_NODES, E, graph.rowptr, graph.sender, graph.receiver, graph.t_rowptr,
                                      graph.t_edge, graph._ws))
    if not args.no_extras:
        # explicit per-edge weights w [E, P, C] (the pages' own interface),
        # same workload; w drawn on the device from a seeded generator
        gen = torch.Generator(device=dev).manual_seed(SEED)
        w_e = torch.randn((E, P, CHANNELS), device=dev, generator=gen)
        wb_e = torch.empty_like(w_e)
        fw = timed(lambda: fc.fc_edge_conv_fwd_w(desc, graph, pos, None, x, w_e, z))
        vw = timed(lambda: fc.fc_edge_conv_vjp_w(desc, graph, pos, None, x, w_e, g, xb, pb, wb_e, ws))
        cw_f, cw_v = compulsory_bytes(N_NODES, E, CHANNELS, n_in, n_out, P, explicit=True)
        out["explicit_weights"] = {
            "fwd_ms": fw, "vjp_ms": vw, "edge_channels_per_s": E * CHANNELS / ((fw + vw) * 1e-3),
            # compulsory bytes: w (and w_bar) streamed once, node arrays once
            "fwd_GBs_compulsory": cw_f / (fw * 1e-3) / 1e9, "vjp_GBs_compulsory": cw_v / (vw * 1e-3) / 1e9,
            "fwd_plus_vjp_frac_hbm_compulsory": (cw_f + cw_v) / ((fw + vw) * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "w_bytes": E * P * CHANNELS * 4}
        # without x_grad the VJP runs receiver-side: w read, w_bar written,
        # each cotangent row read once (compulsory: w, w_bar, g, x, graph,
        # the per-edge position terms written and summed)
        vr = timed(lambda: fc.fc_edge_conv_vjp_w(desc, graph, pos, None, x, w_e, g, None, pb, wb_e, ws))
        cr = 2 * E * P * CHANNELS * 4 + N_NODES * (n_in + n_out) * CHANNELS * 4 + E * 4 * 2 + E * 12 * 3
        out["explicit_weights"]["vjp_pos_w_only_ms"] = vr
        out["explicit_weights"]["vjp_pos_w_only_GBs_compulsory"] = cr / (vr * 1e-3) / 1e9
        # VJP-of-VJP with every cotangent (v_x, v_pos, v_w) and every output
        # (g_hat, x_hat, pos_hat, w_hat); w, v_w and w_hat each move w_bytes
        v_x = torch.randn(x.shape, device=dev, generator=gen)
        v_pos = torch.randn(pos.shape, device=dev, generator=gen)
        v_w = torch.randn((E, P, CHANNELS), device=dev, generator=gen)
        gh, xh, ph = torch.empty_like(g), torch.empty_like(x), torch.empty_like(pos)
        out["explicit_weights"]["vjp_vjp_ms"] = timed(
            lambda: fc.fc_edge_conv_vjp_vjp_w(desc, graph, pos, None, x, w_e, g, v_x, v_pos, v_w, gh, xh, ph, wb_e,
                                              ws))
        del w_e, wb_e, v_w, v_x, v_pos, gh, xh, ph
        # the radial-weight gradient (optional VJP output, a receiver-sorted
        # pass of its own), timed alone and with the rest of the VJP
        Wb = torch.empty_like(W)
        out["breakdown"]["radial_w_grad_ms"] = timed(
            lambda: fc.fc_edge_conv_vjp(desc, graph, pos, None, x, W, g, None, None, Wb, ws))
        out["breakdown"]["vjp_with_radial_w_grad_ms"] = timed(
            lambda: fc.fc_edge_conv_vjp(desc, graph, pos, None, x, W, g, xb, pb, Wb, ws))
        out["extras"] = extras(dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
