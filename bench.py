#!/usr/bin/env python3
"""Throughput of the SO(2) message-passing layer on one MI355X.

One step is one pass of the whole hot path over one synthetic structure,
with inputs already resident in HBM:
  neighbour graph build -> edge geometry (Wigner rows, radial basis) ->
  layer forward (saving activations) -> layer backward -> Hamiltonian blocks
  (edge and on-site) -> the periodic Hamiltonian as one block-sparse row
  structure over the image shifts.
The default workload is the HfO2-like training step: 3,000 atoms (1,000 Hf +
2,000 O) in a 32.8 A periodic cube, cutoff 8 A (~547k directed edges),
lmax 4, mmax 2, C 64, fp32, one layer forward + backward, then the decode
into 13x13 orbital blocks and their assembly into the sparse H(S).
`value` is edges per second of whole steps (wall clock over the timed
steps); the median of per-step HIP-event times is reported beside it, and so
is the step time of as many steps again with the per-launch timing events
off (their cost).  The default run also times, each the same way:
the 8,064-atom GeSbTe-like configuration (bf16 storage, C 128), its 3-layer
forward and its training step (key "gst"); the HfO2-like forward and the
one-GPU-share (halo) forward ("other_configs"); and the saturation sweep of
one layer forward against edge count ("saturation_sweep").  --no-extra
skips them.

Other workloads (--workload): hfo2, halo, gst (forwards; GST is three bf16
layers), gst_train (bf16 training step), hfo2_l6 / hfo2_l8 (forwards at
lmax 6 and 8) and hfo2_l6_train / hfo2_l8_train (their training steps,
without the decode), edge_train (the edge-update block's training step), and m2l /
l2m, which time Matrix -> Label and Label -> Matrix (MALOQ Sec. III-B2,
Fig. 2(c, d)) over a batch of 4,096 small molecules; `value` is atoms per
second there.

Prints one JSON line.  --gpus above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}
FP32_VALU_PEAK_TFLOPS = 78.6   # 256 CU x 4 SIMD x 16 lanes x 2 FLOP x 2.4 GHz (no packed fp32)

WORKLOADS = {
    "train": dict(cfg="train", backward=True, decode=True, layers=1,
                  desc="HfO2-like training step: graph + geometry + 1 layer fwd/bwd + 13x13 blocks + sparse H(S)"),
    "hfo2": dict(cfg="hfo2", backward=False, decode=False, layers=1,
                 desc="HfO2-like forward: graph + geometry + 1 layer fwd"),
    "hfo2_l6": dict(cfg="hfo2_l6", backward=False, decode=False, layers=1,
                    desc="HfO2-like forward at lmax 6 / mmax 2: graph + geometry + 1 layer fwd"),
    "hfo2_l8": dict(cfg="hfo2_l8", backward=False, decode=False, layers=1,
                    desc="HfO2-like forward at lmax 8 / mmax 2: graph + geometry + 1 layer fwd"),
    "hfo2_l6_train": dict(cfg="hfo2_l6", backward=True, decode=False, layers=1,
                          desc="HfO2-like training step at lmax 6 / mmax 2: graph + geometry + 1 layer fwd/bwd"),
    "hfo2_l8_train": dict(cfg="hfo2_l8", backward=True, decode=False, layers=1,
                          desc="HfO2-like training step at lmax 8 / mmax 2: graph + geometry + 1 layer fwd/bwd"),
    "halo": dict(cfg="halo", backward=False, decode=False, layers=1,
                 desc="one GPU's share with ghost halo: graph + geometry + 1 layer fwd"),
    "gst": dict(cfg="gst", backward=False, decode=False, layers=3,
                desc="GeSbTe-like 3-layer forward, bf16 storage"),
    "gst_train": dict(cfg="gst", backward=True, decode=True, layers=1,
                      desc="GeSbTe-like training step, bf16 storage: graph + geometry + 1 layer fwd/bwd + 13x13 blocks "
                           "+ sparse H(S)"),
    "edge_train": dict(cfg="train", backward=True, decode=False, layers=1, edge=True,
                       desc="HfO2-like edge-update block: graph + geometry + edge update fwd/bwd"),
    "m2l": dict(labels="m2l", mols=4096, seed=40,
                desc="Matrix -> Label over 4,096 nabla2DFT-like molecules (10-50 atoms of H C N O F S Cl, "
                     "def2-SVP-like shells, fully connected): orbital layout + labels of every atom and edge"),
    "l2m": dict(labels="l2m", mols=4096, seed=40,
                desc="Label -> Matrix over the same 4,096 molecules: orbital layout + every block written back"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true",
                    help="(train workload) skip the other configurations the default run also measures: the "
                         "GeSbTe-like 3-layer forward and training step, the HfO2-like and one-GPU-share "
                         "forwards, and the saturation sweep")
    ap.add_argument("--workload", default="train", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=500, help="rows of the oracle's timed sample")
    ap.add_argument("--cpu-mols", type=int, default=150, help="molecules of the oracle's timed sample (m2l, l2m)")
    ap.add_argument("--label-order", choices=("src", "dst"), default="dst",
                    help="m2l / l2m: blocks taken per destination atom, or per source atom (the graph's source "
                         "grouping, made before the timed steps)")
    ap.add_argument("--copy-probe-mib", type=int, default=1024,
                    help="size of the plain elementwise copy (y = -x, float32) timed before the steps; it gives "
                         "the measured copy bandwidth, and a counter run sees it as a kernel of known traffic")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="(no GPU) turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script into "
                         "the traffic summary under profiles/ and exit")
    ap.add_argument("--summarize-sq", nargs="+", metavar="PASS_DIR",
                    help="(no GPU) turn two rocprofv3 --pmc runs of this script (the SQ counter sets named in "
                         "the summary it writes) into profiles/sq_<workload>.txt and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="saturation sweep: layer forward and edge geometry time vs edge count, on the first "
                         "rows of the one-GPU-share (halo) graph; prints one JSON line")
    return ap.parse_args()


def grid_of(struct):
    if struct.periodic_mask == 7:
        return np.zeros(3), np.asarray(struct.box, np.float64)
    lo = struct.pos.min(axis=0)
    return lo, (struct.pos.max(axis=0) - lo) * (1 + 1e-12) + 1e-9


class Step:
    """Everything one step needs, allocated once."""

    def __init__(self, wl, dev):
        import torch
        import synth
        import equivariant_gnn_electronic_amd as eg
        self.eg, self.torch = eg, torch
        self.wl = wl
        cfg = self.cfg = synth.CONFIGS[wl["cfg"]]
        s = self.struct = synth.make_structure(cfg)
        x, ws = synth.make_layer_inputs(cfg)
        lo, box = grid_of(s)
        self.pos = torch.from_numpy(s.pos).to(dev)
        g0 = eg.egnn_build_graph(self.pos, s.n_dst, lo, box, s.periodic_mask, s.r_cut)
        self.E = g0.n_edges
        self.builder = eg.GraphBuilder(s.n_dst, s.n_src, lo, box, s.periodic_mask, s.r_cut, self.E, dev)
        self.storage = eg.EGNN_BF16 if cfg.storage == "bf16" else eg.EGNN_F32
        self.desc = eg.layer_desc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut, self.storage)
        dt = torch.bfloat16 if self.storage == eg.EGNN_BF16 else torch.float32
        self.x = torch.from_numpy(x).to(dev).to(dt)
        self.w = [torch.from_numpy(w).to(dev) for w in ws]
        g = self.builder.build(self.pos)
        self.geom = eg.egnn_edge_geom(self.desc, g)
        self.buf = eg.LayerBuffers(self.desc, g, train=wl["backward"])
        K = cfg.K
        # layer outputs; for a stack, ghosts keep their input irreps between layers
        self.xs = [self.x] + [torch.empty((s.n_src, K, cfg.C), dtype=dt, device=dev) for _ in range(wl["layers"])]
        for t in self.xs[1:]:
            t[s.n_dst:] = self.x[s.n_dst:]
        self.edge_out = torch.empty((max(self.E, 1), K, cfg.C), dtype=dt, device=dev) if wl["decode"] else None
        if wl["backward"]:
            self.G = torch.from_numpy(synth.make_cotangent(cfg, s.n_dst)).to(dev)
            self.gx = torch.empty((s.n_src, K, cfg.C), dtype=torch.float32, device=dev)
            self.gw = torch.empty(eg.egnn_layer_weight_count(self.desc), dtype=torch.float32, device=dev)
        if wl.get("edge"):
            self.e = torch.from_numpy(synth.make_edge_embeddings(cfg, self.E)).to(dev).to(dt)
            self.e_out = torch.empty_like(self.e)
            self.Ge = torch.from_numpy(synth.make_edge_cotangent(cfg, self.E)).to(dev)
        if wl["decode"]:
            we, wn = synth.make_decode_weights(cfg)
            self.we = torch.from_numpy(np.concatenate(we)).to(dev)
            self.wn = torch.from_numpy(np.concatenate(wn)).to(dev)

    def __call__(self):
        eg = self.eg
        s = self.struct
        g = self.builder.build(self.pos)
        eg.egnn_edge_geom(self.desc, g, out=self.geom)
        if self.wl.get("edge"):
            eg.egnn_edge_update_fwd(self.desc, g, self.geom, self.w[0], self.xs[0], self.e, e_out=self.e_out,
                                    buffers=self.buf)
            eg.egnn_edge_update_bwd(self.desc, g, self.geom, self.w[0], self.xs[0], self.buf, self.Ge,
                                    grad_x=self.gx, grad_w=self.gw)
            return g
        for i in range(self.wl["layers"]):
            last = i == self.wl["layers"] - 1
            eo = self.edge_out if (last and self.wl["decode"]) else None
            self._fwd(g, i, eo)
        if self.wl["backward"]:
            eg.egnn_layer_bwd(self.desc, g, self.geom, self.w[0], self.xs[0], self.buf, self.G,
                              grad_x=self.gx, grad_w=self.gw)
        if self.wl["decode"]:
            he, hn = eg.egnn_hblocks(self.cfg.lmax, self.cfg.C, self.we, self.wn, self.edge_out[:self.E],
                                     self.xs[-1][:s.n_dst], storage=self.storage)
            # the periodic Hamiltonian: every block in one block-sparse row structure over the image shifts
            eg.egnn_assemble_bsr(g, he, hn)
        return g

    def _fwd(self, g, i, eo):
        import ctypes as ct
        eg = self.eg
        lib = eg._lib.load()
        gs = g.c_struct()
        xin, xout = self.xs[i], self.xs[i + 1]
        eg._lib.check("egnn_layer_fwd", lib.egnn_layer_fwd(
            ct.byref(self.desc), ct.byref(gs), eg._ptr(self.geom), eg._ptr(self.w[i]), eg._ptr(xin),
            eg._ptr(xout), eg._ptr(eo) if eo is not None else None,
            eg._ptr(self.buf.saved) if self.buf.saved is not None else None, eg._ptr(self.buf.ws),
            self.buf.ws.numel(), eg._stream()))


class LabelStep:
    """One pass of Matrix -> Label (or Label -> Matrix) over a batch of molecules,
    inputs resident on the GPU."""

    def __init__(self, wl, dev, by_source=True):
        import torch
        import synth
        import equivariant_gnn_electronic_amd as eg
        self.eg, self.wl = eg, wl
        b = self.batch = synth.make_molecule_batch(wl["seed"], wl["mols"], 10, 50)
        self.basis = eg.Basis(synth.SVP_SHELLS, synth.SVP_MASKS)
        self.mol_ptr = torch.from_numpy(b.mol_ptr).to(dev)
        self.species = torch.from_numpy(b.species).to(dev)
        # the source grouping is made once with the graph (outside the timed steps)
        self.graph = eg.Graph.from_csr(torch.from_numpy(b.row_ptr).to(dev), torch.from_numpy(b.src).to(dev),
                                       group=by_source)
        orb, bad = eg.egnn_orbital_layout(self.basis, self.mol_ptr, self.species)
        assert int(bad.item()) == 0
        self.h_elems = int(orb.mat_off[-1].item())
        self.H = torch.from_numpy(synth.make_matrix_values(wl["seed"] + 1, self.h_elems)).to(dev)
        self.he, self.hn, _ = eg.egnn_matrix_to_label(self.basis, orb, self.graph, self.H)
        self.orb = orb
        self.n_lab = eg.egnn_label_width(self.basis)
        self.E = b.n_edges

    def __call__(self):
        eg = self.eg
        orb, _ = eg.egnn_orbital_layout(self.basis, self.mol_ptr, self.species)
        if self.wl["labels"] == "m2l":
            eg.egnn_matrix_to_label(self.basis, orb, self.graph, self.H)
        else:
            eg.egnn_label_to_matrix(self.basis, orb, self.graph, self.he, self.hn, H=self.H)


def cpu_baseline_labels(wl, n_mols):
    """The fp64 oracle on the first `n_mols` molecules of the same batch (a prefix:
    their atoms, edges and matrices are the first ones of the full arrays)."""
    import synth
    from oracle import labels
    b = synth.make_molecule_batch(wl["seed"], wl["mols"], 10, 50)
    k = min(n_mols, b.n_mols)
    n_at = int(b.mol_ptr[k])
    n_e = int(b.row_ptr[n_at])
    sh, masks = synth.SVP_SHELLS, synth.SVP_MASKS
    src, dst = b.src[:n_e].astype(np.int64), b.dst()[:n_e].astype(np.int64)
    species = b.species[:n_at]
    lay_full = labels.orbital_layout(b.mol_ptr[:k + 1], species, sh, masks)
    H = synth.make_matrix_values(wl["seed"] + 1, lay_full[3][-1]).astype(np.float64)
    t0 = time.perf_counter()
    lay = labels.orbital_layout(b.mol_ptr[:k + 1], species, sh, masks)
    he, hn = labels.matrix_to_labels(H, src, dst, None, species, lay, sh, masks)
    if wl["labels"] == "l2m":
        t0 = time.perf_counter()
        lay = labels.orbital_layout(b.mol_ptr[:k + 1], species, sh, masks)
        labels.labels_to_matrix(he, hn, src, dst, None, species, lay, sh, masks)
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return dict(value=round(n_at / dt, 2), unit="atoms/s", cores=int(threads), kind="oracle",
                sample=f"first {k} molecules of the batch ({n_at} atoms, {n_e} edges), fp64 numpy, {dt:.1f} s")


def run_labels(args, wl, dev):
    import torch
    step = LabelStep(wl, dev, by_source=args.label_order == "src")
    copy_gbs = copy_bandwidth(torch, dev, args.copy_probe_mib)
    eg = step.eg
    ts = timed_steps(torch, eg, step, args.steps, args.warmup)
    ms, med, timing, dropped = ts
    fam, roof = roofline(timing, "f32", args.workload)
    b = step.batch
    kernels = kernel_table(timing, args.steps, copy_gbs)
    name = "Matrix -> Label" if wl["labels"] == "m2l" else "Label -> Matrix"
    out = {
        "metric": f"atoms/s of {name} over a batch of molecules + % of HBM roofline",
        "value": round(b.n_atoms / (ms * 1e-3), 1),
        "unit": "atoms/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded molecule sizes and elements, N(0,1) matrix entries)",
        "config": {"workload": args.workload, "description": wl["desc"], "order": args.label_order,
                   "molecules": b.n_mols,
                   "atoms": b.n_atoms, "edges": step.E, "labels_per_block": step.n_lab,
                   "matrix_entries": step.h_elems,
                   "blocks_per_s": round((b.n_atoms + step.E) / (ms * 1e-3), 1),
                   "median_step_ms": round(med, 4),
                   "ms_per_step_without_kernel_events": round(ts.ms_no_kernel_events, 4)},
        "roofline": dict(kernel=fam, **roof),
        "hbm_copy_gbs": copy_gbs,
        "kernels": kernels,
        "timing_events_dropped": dropped,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_labels(wl, args.cpu_mols)
    print(json.dumps(out), flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "equivariant_gnn_electronic_amd", "csrc")
COPY_KERNEL_TAG = "neg_kernel"


def kernel_source_hash():
    """sha256 over every HIP source and header of the library (a traffic figure is
    only reported for the sources it was measured on)."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")


def read_traffic(workload, family):
    """HBM bytes per launch of `family` from the committed counter summary, or None
    when there is none, it does not cover that kernel, or the sources changed since."""
    try:
        with open(traffic_path(workload)) as fh:
            kv = dict(line.split(": ", 1) for line in fh.read().splitlines() if ": " in line and not line.startswith("#"))
    except OSError:
        return None
    key = f"traffic_bytes_per_launch[{family}]"
    if key not in kv or kv.get("source_sha256") != kernel_source_hash():
        return None
    return float(kv[key])


def _pmc_per_dispatch(d, counter):
    """{dispatch id: (kernel name, value)} from a rocprofv3 csv counter collection."""
    import csv
    import glob
    out = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                k = r["Dispatch_Id"]
                name, v = out.get(k, (r["Kernel_Name"], 0.0))
                out[k] = (name, v + float(r["Counter_Value"]))
    return out


def summarize_traffic(fetch_dir, write_dir, workload, copy_mib, argv):
    """Write profiles/traffic_<workload>.txt: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of each kernel family below, each scaled by the ratio of the known
    bytes of the copy probe to what the same counter read for it."""
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mib * 2 ** 20

    def pick(tab, tag):
        pieces = (tag,) if isinstance(tag, str) else tag
        return [v for name, v in tab.values() if all(t in name for t in pieces)]

    cf, cw = pick(fetch, COPY_KERNEL_TAG), pick(write, COPY_KERNEL_TAG)
    if not cf or not cw:
        raise SystemExit("no copy-probe dispatch in the counter runs")
    sf, sw = copy_bytes / (cf[0] * 1024), copy_bytes / (cw[0] * 1024)
    cmd = (f"python bench.py --workload {workload} --steps 2 --warmup 1 --no-cpu-baseline --no-extra "
           f"--copy-probe-mib {copy_mib}")
    lines = [
        f"# HBM traffic per launch of the main kernels of the {workload} step, from rocprofv3 counters",
        "# made by (from the repository root, on one MI355X):",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <FETCH_DIR> -o run -- {cmd}",
        f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <WRITE_DIR> -o run -- {cmd}",
        f"#   python {' '.join(argv)}",
        f"# copy probe (y = -x, float32): {copy_mib} MiB read + {copy_mib} MiB written; the counters read "
        f"{cf[0]:.0f} KiB fetched, {cw[0]:.0f} KiB written -> scale fetch {sf:.4f}, write {sw:.4f}",
        f"workload: {workload}",
        f"source_sha256: {kernel_source_hash()}",
        f"copy_scale_fetch: {sf:.5f}",
        f"copy_scale_write: {sw:.5f}",
    ]
    for fam, tag in FAMILY_KERNELS.items():
        kf, kw = pick(fetch, tag), pick(write, tag)
        if not kf or len(kf) != len(kw):
            continue
        f_kib, w_kib = float(np.mean(kf)), float(np.mean(kw))
        lines.append(f"# {fam}: {len(kf)} dispatches of {tag if isinstance(tag, str) else ' ... '.join(tag)}; "
                     f"per dispatch FETCH_SIZE {f_kib:.0f} KiB, "
                     f"WRITE_SIZE {w_kib:.0f} KiB")
        lines.append(f"traffic_bytes_per_launch[{fam}]: {(f_kib * sf + w_kib * sw) * 1024:.0f}")
    os.makedirs(os.path.dirname(traffic_path(workload)), exist_ok=True)
    with open(traffic_path(workload), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SQ_PASS1 = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
            "SQ_INSTS_VALU", "SQ_ACTIVE_INST_ANY")
SQ_PASS2 = ("GRBM_GUI_ACTIVE", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
            "SQ_ACTIVE_INST_LDS", "SQ_INST_CYCLES_VMEM", "SQ_WAIT_INST_LDS")
SQ_PASS3 = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES")


def summarize_sq(d1, d2, workload, argv, d3=None):
    """profiles/sq_<workload>.txt: per kernel, instruction mix per wave and the
    VALU issue fraction = SQ_INSTS_VALU x 4 cycles (a wave64 VALU instruction on a
    16-lane SIMD) / (1024 SIMDs x the kernel's cycles, GRBM_GUI_ACTIVE / 8 XCDs)."""
    import collections
    import csv
    import glob
    import re

    def load(d):
        per = collections.defaultdict(collections.Counter)
        meta = {}
        span = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                k = (path, r["Dispatch_Id"])
                per[k][r["Counter_Name"]] += float(r["Counter_Value"])
                meta[k] = (r["Kernel_Name"], r["VGPR_Count"], r["Accum_VGPR_Count"], r["LDS_Block_Size"])
                if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                    span[k] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        by = collections.defaultdict(collections.Counter)
        n = collections.Counter()
        m = {}
        for k, c in per.items():
            by[meta[k][0]].update(c)
            by[meta[k][0]]["_ns"] += span.get(k, 0)
            n[meta[k][0]] += 1
            m[meta[k][0]] = meta[k]
        return by, n, m

    a, na, ma = load(d1)
    b, _, _ = load(d2)
    c3 = load(d3)[0] if d3 else {}
    cmd = f"python bench.py --workload {workload} --steps 2 --warmup 1 --no-cpu-baseline --no-extra --copy-probe-mib 256"
    lines = [f"# SQ counters per kernel of the {workload} step (sums over every dispatch of the run), from rocprofv3",
             "# made by (from the repository root, on one MI355X):",
             f"#   rocprofv3 --pmc {' '.join(SQ_PASS1)} --output-format csv -d <PASS1_DIR> -o run -- {cmd}",
             f"#   rocprofv3 --pmc {' '.join(SQ_PASS2)} --output-format csv -d <PASS2_DIR> -o run -- {cmd}",
             *([f"#   rocprofv3 --pmc {' '.join(SQ_PASS3)} --output-format csv -d <PASS3_DIR> -o run -- {cmd}",
                "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 256 CUs * 4 SIMDs), both from pass 3"]
               if d3 else []),
             f"#   python {' '.join(argv)}",
             "# valu_issue = SQ_INSTS_VALU * 4 / (1024 * GRBM_GUI_ACTIVE / 8): the fraction of SIMD cycles issuing VALU",
             "# (wave64 on 16-lane SIMDs; GRBM_GUI_ACTIVE summed over the 8 XCDs); per-wave figures are means;",
             "# clock = GRBM_GUI_ACTIVE / 8 over the dispatches' time (End - Start), the shader clock the kernel ran at",
             f"workload: {workload}"]
    rows = []
    for name, c in a.items():
        gui = b.get(name, {}).get("GRBM_GUI_ACTIVE", 0.0)
        if gui < 1e6 or c["SQ_WAVES"] <= 0:
            continue
        rows.append((gui, name, c, b.get(name, collections.Counter())))
    rows.sort(key=lambda r: -r[0])
    for gui, name, c, c2 in rows[:16]:
        short = name.replace("egnn::(anonymous namespace)::", "").replace("void ", "")
        mt = re.match(r"([A-Za-z0-9_:]+)(<[^(]*>)?", short)
        short = (mt.group(1) + (mt.group(2) or "")) if mt else short[:80]
        w = c["SQ_WAVES"]
        wc = c["SQ_WAVE_CYCLES"]
        vg, ag, lds = ma[name][1:]
        ns = c2.get("_ns", 0)
        clk = f"  clock {gui / 8 / ns:.2f} GHz" if ns > 0 else ""
        lines.append(f"kernel: {short}  dispatches {na[name]}  vgpr {vg} agpr {ag} lds {lds} B{clk}")
        lines.append(f"  per wave: VALU {c['SQ_INSTS_VALU'] / w:.0f}, VMEM rd {c2['SQ_INSTS_VMEM_RD'] / w:.0f}, "
                     f"VMEM wr {c2['SQ_INSTS_VMEM_WR'] / w:.0f}, LDS {c2['SQ_INSTS_LDS'] / w:.0f}, "
                     f"SALU {c2['SQ_INSTS_SALU'] / w:.0f}, wave cycles {wc / w:.0f}")
        lines.append(f"  valu_issue {c['SQ_INSTS_VALU'] * 4 / (1024 * gui / 8):.3f}; of wave cycles: active VALU "
                     f"{c['SQ_ACTIVE_INST_VALU'] / wc:.3f}, active any {c['SQ_ACTIVE_INST_ANY'] / wc:.3f}, "
                     f"waiting (any) {c['SQ_WAIT_ANY'] / wc:.3f}, waiting to issue {c['SQ_WAIT_INST_ANY'] / wc:.3f}, "
                     f"active LDS {c2['SQ_ACTIVE_INST_LDS'] / wc:.3f}")
        m3 = c3.get(name) if d3 else None
        if m3 and m3.get("GRBM_GUI_ACTIVE", 0) > 0:
            lines.append(f"  mfma_busy {m3['SQ_VALU_MFMA_BUSY_CYCLES'] / (m3['GRBM_GUI_ACTIVE'] / 8 * 1024):.3f}")
    path = os.path.join(ROOT, "profiles", f"sq_{workload}.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# timing family -> piece (or pieces, all present) of its kernel's symbol name
FAMILY_KERNELS = {
    # kernel-name pieces ("::" keeps gemm from matching cgemm; the GEMM templates carry
    # tile widths after these arguments)
    "cgemm_dw_f32": "::cgemm_f32_kernel<false, false, false,",
    "cgemm_fwd_f32": "::cgemm_f32_kernel<true, true, true,",
    "cgemm_dx_f32": "::cgemm_f32_kernel<true, false, true,",
    "gemm_tn_f32": "::gemm_f32_kernel<false, false,",
    "gemm_nt_f32": "::gemm_f32_kernel<true, true,",
    "gemm_nn_f32": "::gemm_f32_kernel<true, false,",
    "gemm_nt_bf16": "gemm_bf16_lds_kernel",  # forward and input-gradient launches alike
    "gemm_dw_bf16": "gemm_bf16_tn_kernel",
    "rotate_in": "::scatter_in_",
    "aggregate": "::aggregate_",
    "hblocks": "hblocks_kernel",
    "assemble_bsr": "::bsr_values_kernel",   # the value copy (the index pass moves ~15 B per block)
    "edge_update": "::edge_update_kernel<",
    "edge_dy": "::edge_dy_kernel<",
    "matrix_to_label": ("::labels_kernel<", ", true>"),   # every (chunk, pass) instantiation
    "label_to_matrix": ("::labels_kernel<", ", false>"),
}


def roofline(timing, dtype, workload):
    """Dominant kernel family by total time, with its achieved rate against the peak."""
    fam, t = max(timing.items(), key=lambda kv: kv[1]["total_ms"])
    per_launch_ms = t["total_ms"] / t["launches"]
    if t["flops"] > 0:
        achieved = t["flops"] / t["launches"] / (per_launch_ms * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS["bf16" if "bf16" in fam else "f32"]
        r = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                 frac=round(achieved / peak, 4), traffic=read_traffic(workload, fam))
        if fam.startswith("cgemm"):
            # the complex products run as three real GEMMs: 3/4 of the algorithmic FLOPs execute
            r["executed_frac"] = round(0.75 * achieved / peak, 4)
        return fam, r
    achieved = t["bytes"] / t["launches"] / (per_launch_ms * 1e-3) / 1e9
    return fam, dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                     frac=round(achieved / HBM_PEAK_GBS, 4), traffic=read_traffic(workload, fam))


def cpu_baseline(wl, rows_n):
    """The fp64 oracle on a sample of destination rows of the same structure.

    The sampled rows become the first rows of a relabelled problem (all atoms
    stay sources), so the oracle does exactly the per-edge work of the full
    step for the sampled rows' edges: brute-force neighbour rows, layer
    forward, backward and decode.
    """
    import synth
    from oracle import decode, layer, neighbors
    cfg = synth.CONFIGS[wl["cfg"]]
    s = synth.make_structure(cfg)
    x, ws = synth.make_layer_inputs(cfg)
    rows = np.sort(np.random.default_rng(0).choice(s.n_dst, min(rows_n, s.n_dst), replace=False))
    perm = np.concatenate([rows, np.setdiff1d(np.arange(s.n_src), rows)])
    pos, xp = s.pos[perm], x[perm].astype(np.float64)
    d = layer.LayerDesc(cfg.lmax, cfg.mmax, cfg.C, cfg.n_rbf, cfg.r_cut)
    t0 = time.perf_counter()
    g = neighbors.build_graph(pos, len(rows), s.box, s.periodic_mask, s.r_cut)
    if wl.get("edge"):
        e = synth.make_edge_embeddings(cfg, len(g["src"])).astype(np.float64)
        f = layer.edge_update_forward(g, xp, e, ws[0].astype(np.float64), d)
        layer.edge_update_backward(g, xp, ws[0].astype(np.float64), d, f, np.ones_like(e))
        dt = time.perf_counter() - t0
        E = len(g["src"])
        return dict(value=round(E / dt, 2), unit="edges/s", cores=len(os.sched_getaffinity(0)), kind="oracle",
                    sample=f"{len(rows)} destination rows ({E} edges) of the same structure, fp64 numpy, {dt:.1f} s")
    xl = xp
    for i in range(wl["layers"]):
        f = layer.layer_forward(g, xl, ws[i].astype(np.float64), d)
        xl = np.concatenate([f["x_out"], xl[len(rows):]])
    if wl["backward"]:
        G = synth.make_cotangent(cfg, s.n_dst)[rows].astype(np.float64)
        layer.layer_backward(g, xp, ws[0].astype(np.float64), d, f, G)
    if wl["decode"]:
        we, wn = synth.make_decode_weights(cfg)
        decode.hblocks(f["edge_out"], we)
        decode.hblocks(f["x_out"], wn)
    dt = time.perf_counter() - t0
    E = len(g["src"])
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return dict(value=round(E / dt, 2), unit="edges/s", cores=int(threads), kind="oracle",
                sample=f"{len(rows)} destination rows ({E} edges) of the same structure, fp64 numpy, "
                       f"{dt:.1f} s")


def copy_bandwidth(torch, dev, mib):
    """Measured HBM rate of a plain elementwise copy (y = -x, float32, `mib` MiB
    read and written), GB/s counting both directions; a practical ceiling beside
    the 8 TB/s peak."""
    n = mib * 2 ** 20 // 4
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    ms = _median_ms(torch, lambda: torch.neg(x, out=y), 2, 10)
    del x, y
    torch.cuda.empty_cache()
    return round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)


def _median_ms(torch, fn, warmup, reps):
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def sweep(dev, warmup, reps):
    """Edges/s of one layer forward (and of the edge geometry alone) against the
    edge count, from 10^3 edges to the whole 3.2M-edge halo graph.  Each point
    takes the first rows of the destination-sorted graph, so its edges are a
    prefix of the full arrays; the time is the median of `reps` runs."""
    import torch
    st = Step(dict(cfg="halo", backward=False, decode=False, layers=1, desc=""), dev)
    eg = st.eg
    g = st.builder.build(st.pos)
    row_ptr = g.row_ptr.cpu().numpy()
    points = []
    targets = [1e3, 3e3, 1e4, 3e4, 1e5, 3e5, 1e6, 2e6, float(st.E)]
    for tgt in targets:
        r = int(min(np.searchsorted(row_ptr, tgt), g.n_dst))
        E = int(row_ptr[r])
        # the source grouping must describe exactly the prefix's edges (the forward walks it)
        src = g.src[:E].cpu().numpy()
        perm = np.argsort(src, kind="stable").astype(np.int32)
        sptr = np.concatenate([[0], np.cumsum(np.bincount(src, minlength=g.n_src))]).astype(np.int32)
        sub = eg.Graph(r, g.n_src, E, g.row_ptr[:r + 1].clone(), g.src[:E].clone(), g.shift[:E].clone(),
                       g.vec[:E].clone(), g.dist[:E].clone(), torch.from_numpy(sptr).to(dev),
                       torch.from_numpy(perm).to(dev))
        assert sub.src_ptr.numel() == g.n_src + 1 and int(sptr[-1]) == E == sub.src.numel()
        geom = eg.egnn_edge_geom(st.desc, sub)
        buf = eg.LayerBuffers(st.desc, sub, train=False)
        xout = torch.empty((max(r, 1), st.cfg.K, st.cfg.C), dtype=torch.float32, device=dev)
        t_geom = _median_ms(torch, lambda: eg.egnn_edge_geom(st.desc, sub, out=geom), warmup, reps)
        t_layer = _median_ms(torch, lambda: eg.egnn_layer_fwd(st.desc, sub, geom, st.w[0], st.x, x_out=xout,
                                                              buffers=buf), warmup, reps)
        points.append(dict(rows=r, edges=E, layer_ms=round(t_layer, 4), edges_per_s=round(E / t_layer * 1e3, 1),
                           geom_ms=round(t_geom, 4), geom_edges_per_s=round(E / t_geom * 1e3, 1)))
        print(f"sweep E={E} layer {t_layer:.3f} ms geom {t_geom:.3f} ms", file=sys.stderr, flush=True)
    return dict(metric="edges/s of one layer forward vs edge count (saturation sweep)", unit="edges/s",
                n_gpus=1, warmup=warmup, reps=reps, dtype="f32", data="synthetic",
                config={"workload": "halo prefix", "lmax": st.cfg.lmax, "mmax": st.cfg.mmax, "C": st.cfg.C},
                points=points)


class TimedSteps(tuple):
    """(wall ms per step, median event ms per step, timing, dropped), plus
    `.ms_no_kernel_events`: the wall ms per step of the same number of steps run
    again right after, with the per-launch events off (their cost = the difference)."""
    ms_no_kernel_events = None


def timed_steps(torch, eg, step, steps, warmup):
    """Run `warmup` untimed steps, then `steps` timed ones with per-launch HIP-event
    timing on (egnn_timing_*) and one pair of events around each step on the launch
    stream.  Then the same number of steps again with the per-launch events off,
    outside the timed region, to state what the events cost."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    eg.egnn_timing_reset()
    eg.egnn_timing_enable(True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eg.egnn_timing_enable(False)
    timing, dropped = eg.egnn_timing_collect()
    med = float(np.median([a.elapsed_time(b) for a, b in ev]))
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    out = TimedSteps(((t1 - t0) * 1e3 / steps, med, timing, dropped))
    out.ms_no_kernel_events = (t3 - t2) * 1e3 / steps
    return out


def kernel_table(timing, steps, copy_gbs):
    """Per timing family: launches and ms per step, rate, and the fraction of the
    MFMA peak of its dtype (GEMM families) or of the HBM peak and the measured copy."""
    kernels = {}
    for k, v in sorted(timing.items(), key=lambda kv: -kv[1]["total_ms"]):
        sec = v["total_ms"] * 1e-3
        gbs = v["bytes"] / sec / 1e9 if v["bytes"] > 0 else None
        kernels[k] = dict(launches_per_step=v["launches"] / steps, ms_per_step=round(v["total_ms"] / steps, 4),
                          tflops=round(v["flops"] / sec / 1e12, 2) if v["flops"] > 0 else None,
                          algorithmic_gbs=round(gbs, 1) if gbs else None)
        if v["flops"] > 0:
            peak = MFMA_PEAK_TFLOPS["bf16" if "bf16" in k else "f32"]
            kernels[k]["mfma_frac"] = round(v["flops"] / sec / 1e12 / peak, 4)
        elif gbs:
            kernels[k]["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
            if copy_gbs:
                kernels[k]["copy_frac"] = round(gbs / copy_gbs, 4)
    return kernels


def extra_workloads(torch, dev, names, steps, warmup, copy_gbs):
    """Other configurations timed like the headline step, each with its own
    per-family roofline fractions: {name: result}."""
    out = {}
    for name in names:
        wl = WORKLOADS[name]
        step = Step(wl, dev)
        ts = timed_steps(torch, step.eg, step, steps, warmup)
        ms, med, timing, dropped = ts
        L = wl["layers"]
        fam, roof = roofline(timing, "bf16" if step.cfg.storage == "bf16" else "f32", name)
        out[name] = {
            "description": wl["desc"], "edges": step.E, "atoms": step.struct.n_dst, "layers": L,
            "ms_per_step": round(ms, 3), "median_step_ms": round(med, 3),
            "ms_per_step_without_kernel_events": round(ts.ms_no_kernel_events, 3),
            "edges_per_s_per_layer": round(step.E * L / (ms * 1e-3), 1),
            "edges_per_s_per_layer_median": round(step.E * L / (med * 1e-3), 1),
            "nodes_per_s_per_layer": round(step.struct.n_dst * L / (ms * 1e-3), 1),
            "roofline": dict(kernel=fam, **roof), "kernels": kernel_table(timing, steps, copy_gbs),
            "timing_events_dropped": dropped}
        print(f"[bench] {name}: {ms:.3f} ms per step", file=sys.stderr, flush=True)
        del step
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], args.workload,
                          args.copy_probe_mib, sys.argv)
        return
    if args.summarize_sq:
        if len(args.summarize_sq) not in (2, 3):
            raise SystemExit("--summarize-sq takes PASS1_DIR PASS2_DIR [PASS3_DIR]")
        summarize_sq(*args.summarize_sq[:2], args.workload, sys.argv,
                     args.summarize_sq[2] if len(args.summarize_sq) == 3 else None)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU path is not built",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.sweep:
        print(json.dumps(sweep(dev, max(args.warmup, 5), max(args.steps, 20))), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if "labels" in wl:
        run_labels(args, wl, dev)
        return
    step = Step(wl, dev)
    copy_gbs = copy_bandwidth(torch, dev, args.copy_probe_mib)
    ts = timed_steps(torch, step.eg, step, args.steps, args.warmup)
    ms, med, timing, dropped = ts
    E = step.E
    cfg = step.cfg
    dtype = "bf16" if cfg.storage == "bf16" else "f32"
    fam, roof = roofline(timing, dtype, args.workload)
    kernels = kernel_table(timing, args.steps, copy_gbs)
    out = {
        "metric": "edges/s per SO(2) message-passing layer (fwd+bwd) + % of HBM/MFMA roofline",
        "value": round(E * wl["layers"] / (ms * 1e-3), 1),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded RSA structure, N(0,1) irreps, N(0,1/fan_in) weights)",
        "config": {"workload": args.workload, "description": wl["desc"], "atoms": step.struct.n_dst,
                   "sources": step.struct.n_src, "edges": E, "lmax": cfg.lmax, "mmax": cfg.mmax, "C": cfg.C,
                   "layers": wl["layers"], "r_cut": cfg.r_cut, "storage": cfg.storage,
                   "nodes_per_s": round(step.struct.n_dst * wl["layers"] / (ms * 1e-3), 1),
                   "ms_per_layer": round(ms / wl["layers"], 3),
                   "median_step_ms": round(med, 3),
                   "edges_per_s_median": round(E * wl["layers"] / (med * 1e-3), 1),
                   "ms_per_step_without_kernel_events": round(ts.ms_no_kernel_events, 3)},
        "roofline": dict(kernel=fam, **roof),
        "hbm_copy_gbs": copy_gbs,
        "kernels": kernels,
        "timing_events_dropped": dropped,
    }
    if args.workload == "train" and not args.no_extra:
        del step
        torch.cuda.empty_cache()
        ex = extra_workloads(torch, dev, ("gst", "gst_train", "hfo2", "halo"), args.steps, args.warmup, copy_gbs)
        out["gst"] = {"forward_3_layers": ex["gst"], "train_step": ex["gst_train"]}
        out["other_configs"] = {"hfo2_forward": ex["hfo2"], "halo_forward": ex["halo"]}
        out["saturation_sweep"] = sweep(dev, 5, 20)["points"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
