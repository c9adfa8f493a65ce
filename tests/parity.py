"""Helpers shared by the GPU parity tests: run the library and the oracle on
the same inputs and measure the worst slice error (normwise for out and M,
per element for z)."""

import numpy as np
import torch

import oracle
import synth

BF16_TOL = 2e-2
F32_TOL = 1e-4


def tolerance(dtype):
    return F32_TOL if dtype == torch.float32 else BF16_TOL


def unit_inputs(inp, b, j, G):
    """float64 host copies of one (batch, KV head) unit's inputs, with
    leading dimensions of size 1 so the oracle sees B = Hkv = 1."""
    sl = slice(j * G, (j + 1) * G)
    return dict(
        q=synth.to_f64(inp["q"][b:b + 1, sl]),
        k=synth.to_f64(inp["k"][b:b + 1, j:j + 1]),
        v=synth.to_f64(inp["v"][b:b + 1, j:j + 1]),
        beta=synth.to_f64(inp["beta"][sl]),
        M0=synth.to_f64(inp["M0"][b:b + 1, j:j + 1]),
        z0=synth.to_f64(inp["z0"][b:b + 1, j:j + 1]),
    )


def compare_units(inp, result, seg_len, rule, units, out_segments=None):
    """Run the oracle on each (b, j) of ``units`` and return the worst errors
    (out, M_final, z_final) of the GPU result over those units."""
    out, M, z = result
    Hq, Hkv = inp["q"].shape[1], inp["k"].shape[1]
    G = Hq // Hkv
    worst = [0.0, 0.0, 0.0]
    for b, j in units:
        u = unit_inputs(inp, b, j, G)
        ro, rM, rz = oracle.forward(u["q"], u["k"], u["v"], u["beta"], u["M0"], u["z0"],
                                    seg_len, rule, out_segments=out_segments)
        go = synth.to_f64(out[b:b + 1, j * G:(j + 1) * G])
        gM = synth.to_f64(M[b:b + 1, j:j + 1])
        gz = synth.to_f64(z[b:b + 1, j:j + 1])
        worst[0] = max(worst[0], oracle.slice_errors(go, ro))
        worst[1] = max(worst[1], oracle.slice_errors(gM, rM))
        worst[2] = max(worst[2], oracle.slice_errors(gz, rz, elementwise=True))
    return tuple(worst)


def all_units(B, Hkv):
    return [(b, j) for b in range(B) for j in range(Hkv)]


def random_inputs(B, Hq, Hkv, L, d, dtype, device, seed=0, m0_scale=0.0, z0=1e-6, dv=None):
    """Seeded Gaussian inputs; ``dv`` gives v (and M0's columns) another width."""
    dv = d if dv is None else dv
    g = torch.Generator(device="cpu").manual_seed(seed)
    mk = lambda *s: torch.randn(*s, generator=g, dtype=torch.float32)
    inp = dict(
        q=mk(B, Hq, L, d).to(dtype), k=mk(B, Hkv, L, d).to(dtype), v=mk(B, Hkv, L, dv).to(dtype),
        beta=mk(Hq), M0=m0_scale * mk(B, Hkv, d, dv),
        z0=(torch.full((B, Hkv, d), z0) if m0_scale == 0.0
            else 0.5 + torch.rand(B, Hkv, d, generator=g)),
    )
    return {k: v.to(device).contiguous() for k, v in inp.items()}


def _unit_errors(task):
    """Pool worker: the oracle on one unit of workload ``w`` (inputs drawn on
    the CPU from the per-slice seeds) against the GPU result stored in the
    files under ``prefix``; returns the unit's (out, M, z) errors."""
    import threadpoolctl

    w, rule, b, j, prefix, out_segments = task
    with threadpoolctl.threadpool_limits(1):
        u = synth.make_unit_inputs(w, b, j)
        ro, rM, rz = oracle.forward(u["q"], u["k"], u["v"], u["beta"], u["M0"], u["z0"],
                                    w.seg_len, rule, out_segments=out_segments)
        G = w.Hq // w.Hkv
        out = np.load(prefix + "out.npy", mmap_mode="r")
        go = out[b:b + 1, j * G:(j + 1) * G]
        if go.dtype == np.uint16:  # bfloat16 bits
            go = (go.astype(np.uint32) << 16).view(np.float32)
        M = np.load(prefix + "M.npy", mmap_mode="r")[b:b + 1, j:j + 1]
        z = np.load(prefix + "z.npy", mmap_mode="r")[b:b + 1, j:j + 1]
        return (oracle.slice_errors(np.asarray(go, dtype=np.float64), ro),
                oracle.slice_errors(np.asarray(M, dtype=np.float64), rM),
                oracle.slice_errors(np.asarray(z, dtype=np.float64), rz, elementwise=True))


def compare_units_pool(w, rule, result, units, procs=16, out_segments=None):
    """compare_units for a workload whose inputs were made on the CPU by
    synth.make_inputs(w, "cpu") (and copied to the GPU): the oracle runs on
    each unit in a pool of worker processes (started by spawn, one BLAS thread
    each), reading the GPU result from files in /dev/shm. Returns the worst
    (out, M_final, z_final) errors over the units."""
    import multiprocessing
    import os
    import tempfile

    import torch

    out, M, z = result
    tmp = tempfile.mkdtemp(prefix="infini_parity_", dir="/dev/shm" if os.path.isdir("/dev/shm")
                           else None)
    prefix = os.path.join(tmp, "")
    try:
        o = out.detach().cpu()
        np.save(prefix + "out.npy", o.view(torch.int16).numpy().view(np.uint16)
                if o.dtype == torch.bfloat16 else o.float().numpy())
        np.save(prefix + "M.npy", M.detach().cpu().numpy())
        np.save(prefix + "z.npy", z.detach().cpu().numpy())
        n = max(1, min(procs, len(units), os.cpu_count() or 1))
        with multiprocessing.get_context("spawn").Pool(n) as pool:
            errs = pool.map(_unit_errors, [(w, rule, b, j, prefix, out_segments)
                                           for b, j in units], chunksize=1)
    finally:
        for f in ("out.npy", "M.npy", "z.npy"):
            try:
                os.remove(prefix + f)
            except OSError:
                pass
        os.rmdir(tmp)
    return tuple(max(e[k] for e in errs) for k in range(3))
