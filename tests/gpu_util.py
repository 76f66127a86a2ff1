"""Helpers for GPU parity tests: device upload, the HIP call, oracle comparison."""
import os
import sys

import numpy as np

from delta_rule_recurrent_kda_amd import inputs

# fp32 inputs: relative Frobenius error per (sample, head) block of O and of S.
TOL_F32_FROB = 1e-4
# bf16 inputs: per output row max|err| <= 2e-2 * ||row_ref||; same per key-channel row of S.
TOL_BF16_ROW = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(spec, a, device="cuda:0"):
    import torch
    dt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    out = {}
    for name in ("q", "k", "v", "log_alpha", "beta"):
        arr = a[name]
        if spec.dtype == "bf16":
            t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(arr)
        out[name] = t.to(device).contiguous()
        assert out[name].dtype == dt
    out["cu_seqlens"] = torch.from_numpy(a["cu_seqlens"].astype(np.int32)).to(device)
    return out


def run_hip(spec, d, stream=None, initial_state=None, qk_l2norm=False):
    """Call the library through the C ABI; returns fp64 numpy (out, final_state)."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    o, fs = kda.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"],
                        stream=stream, initial_state=initial_state, qk_l2norm=qk_l2norm)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), fs.cpu().double().numpy()


def oracle_ref(spec, a, heads=None, threads=None, initial_state=None, qk_l2norm=False):
    import oracle
    f = {x: inputs.to_f64(a[x], spec.dtype) for x in ("q", "k", "v", "log_alpha", "beta")}
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    return oracle.forward(f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], a["cu_seqlens"],
                          heads=heads, threads=threads, initial_state=initial_state,
                          qk_l2norm=qk_l2norm)


def unnormalised(spec, a, seed):
    """The same draws with every (token, head) q and k vector scaled by its own factor
    in [0.05, 20], and a few of them set to zero, re-stored in the spec's dtype."""
    rng = np.random.default_rng(seed)
    T, H = spec.total_tokens, spec.heads
    b = dict(a)
    for i, x in enumerate(("q", "k")):
        f = inputs.to_f64(a[x], spec.dtype) * rng.uniform(0.05, 20.0, (T, H, 1))
        for t in (1 + i, T // 2 + i, T - 1 - i):
            if 0 <= t < T:
                f[t, t % H] = 0.0
        b[x] = inputs.f64_to_bf16_bits(f) if spec.dtype == "bf16" else f.astype(np.float32)
    return b


def compare(spec, out, fs, o_ref, f_ref, heads=None, label=""):
    """Assert the tolerance for spec.dtype; returns a dict of error figures."""
    hs = list(range(spec.heads)) if heads is None else list(heads)
    cu = spec.cu_seqlens()
    o, orf = out[:, hs], o_ref[:, hs]
    s, srf = fs[:, hs], f_ref[:, hs]
    stats = {}
    if spec.dtype == "f32":
        worst_o = worst_s = 0.0
        for n in range(len(cu) - 1):
            seg = slice(cu[n], cu[n + 1])
            for j in range(len(hs)):
                ref = orf[seg, j]
                nr = np.linalg.norm(ref)
                e = np.linalg.norm(o[seg, j] - ref) / nr if nr > 0 else np.abs(o[seg, j]).max(initial=0)
                worst_o = max(worst_o, e)
                nr = np.linalg.norm(srf[n, j])
                e = np.linalg.norm(s[n, j] - srf[n, j]) / nr if nr > 0 else np.abs(s[n, j]).max()
                worst_s = max(worst_s, e)
        stats.update(frob_out=worst_o, frob_state=worst_s)
        log(f"[{label}] f32 worst per-block rel frob: out {worst_o:.3e} state {worst_s:.3e}")
        assert worst_o <= TOL_F32_FROB and worst_s <= TOL_F32_FROB, stats
        return stats
    rown = np.linalg.norm(orf, axis=2)
    rowe = np.abs(o - orf).max(axis=2)
    zero = rown == 0
    assert np.all(rowe[zero] == 0), "rows with a zero reference must be exactly zero"
    rel = np.where(zero, 0.0, rowe / np.where(zero, 1.0, rown))
    if rel.size == 0:                   # a pack with no tokens: only the final states to compare
        rel = np.zeros((1, 1))
        rown = np.zeros((1, 1))
    i = np.unravel_index(np.argmax(rel), rel.shape)
    srn = np.linalg.norm(srf, axis=3)
    sre = np.abs(s - srf).max(axis=3)
    szero = srn == 0
    assert np.all(sre[szero] == 0)
    srel = np.where(szero, 0.0, sre / np.where(szero, 1.0, srn))
    frob = np.linalg.norm(o - orf) / max(np.linalg.norm(orf), 1e-300) if orf.size else 0.0
    stats.update(worst_row=float(rel.max()), worst_row_at=(int(i[0]), hs[int(i[1])]),
                 worst_row_norm=float(rown[i]), median_row=float(np.median(rel)),
                 worst_state_row=float(srel.max()), frob_out=float(frob))
    log(f"[{label}] bf16 worst row rel {rel.max():.3e} at token {i[0]} head {hs[i[1]]} "
        f"(ref norm {rown[i]:.3e}), median {np.median(rel):.3e}, state row {srel.max():.3e}, "
        f"frob {frob:.3e}")
    assert rel.max() <= TOL_BF16_ROW and srel.max() <= TOL_BF16_ROW, stats
    return stats
