"""HIP path vs the fp64 oracle on seeded inputs (GPU; calls go through the C ABI)."""
import numpy as np
import pytest

from delta_rule_recurrent_kda_amd import inputs

import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from delta_rule_recurrent_kda_amd import kda
    kda.library()


def _check(spec, heads=None, label=None):
    label = label or spec.name
    gu.log(f"case {label}: seqs={len(spec.seq_lens)} T={spec.total_tokens} H={spec.heads} "
           f"dk={spec.dk} dv={spec.dv} {spec.dtype}")
    a = inputs.generate(spec)
    d = gu.device_inputs(spec, a)
    out, fs = gu.run_hip(spec, d)
    o_ref, f_ref = gu.oracle_ref(spec, a, heads=heads)
    return gu.compare(spec, out, fs, o_ref, f_ref, heads=heads, label=label)


EDGE = [
    ("L1", [1], 2, 128, 128, "bf16"),
    ("L17", [17], 2, 128, 128, "bf16"),
    ("L64", [64], 2, 128, 128, "bf16"),
    ("L65", [65], 2, 128, 128, "bf16"),
    ("L129_ragged_many", [129, 3, 64, 200, 1, 63], 3, 128, 128, "bf16"),
    ("zero_len", [0, 50, 0, 0, 77, 0], 2, 128, 128, "bf16"),
    ("tiny_pack100", list(np.random.default_rng(5).integers(1, 21, 100)), 2, 128, 128, "bf16"),
    ("d64_bf16", [300, 45], 3, 64, 64, "bf16"),
    ("dk64_dv128", [150, 99], 2, 64, 128, "bf16"),
    ("dk128_dv64", [150, 99], 2, 128, 64, "bf16"),
    ("f32_d128", [33, 100, 1, 257], 2, 128, 128, "f32"),
    ("f32_d64_ragged", [31, 32, 33, 95], 2, 64, 64, "f32"),
    ("f32_dk64_dv128", [70, 10], 1, 64, 128, "f32"),
]


@pytest.mark.parametrize("name,lens,H,dk,dv,dt", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, lens, H, dk, dv, dt):
    spec = inputs.KdaSpec(name, tuple(int(x) for x in lens), H, dk, dv, dt, (0.001, 0.1), 4242)
    _check(spec, label=name)


def test_strong_decay_within_precondition():
    spec = inputs.KdaSpec("strong", (300, 129), 2, 128, 128, "bf16", (0.3, 1.2), 77)
    _check(spec, label="strong decay")


def test_beta_zero_gives_exact_zeros():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    spec = inputs.custom([100, 37], heads=2, d=128, seed=3)
    a = inputs.generate(spec)
    a["beta"][:] = 0
    d = gu.device_inputs(spec, a)
    o, fs = kda.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(o.float()).item() == 0
    assert torch.count_nonzero(fs).item() == 0


def test_nan_stays_in_its_sample_and_head():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    spec = inputs.custom([80, 80, 80], heads=2, d=128, seed=4)
    a = inputs.generate(spec)
    a["v"][90, 1, 5] = 0x7FC0                     # NaN in sample 1, head 1
    d = gu.device_inputs(spec, a)
    o, fs = kda.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"])
    torch.cuda.synchronize()
    bad = torch.isnan(o.float()).any(dim=2).cpu().numpy()
    assert not bad[:80].any() and not bad[160:].any() and not bad[:, 0].any()
    assert bad[90:160, 1].all()
    fsn = torch.isnan(fs).cpu().numpy()
    assert fsn[1, 1].any() and not fsn[[0, 2]].any() and not fsn[1, 0].any()


def test_bitwise_deterministic():
    import torch
    spec = inputs.custom([700, 300], heads=4, d=128, seed=6)
    a = inputs.generate(spec)
    d = gu.device_inputs(spec, a)
    from delta_rule_recurrent_kda_amd import kda
    o1, f1 = kda.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"])
    o2, f2 = kda.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(f1, f2)


def test_side_stream_and_null_final_state():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    spec = inputs.custom([130, 70], heads=2, d=128, seed=8)
    a = inputs.generate(spec)
    d = gu.device_inputs(spec, a)
    ref, _ = kda.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"])
    s = torch.cuda.Stream()
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        kda.kda_forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"], out, None,
                        stream=s)
    s.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_named_config_full(cfg):
    _check(inputs.config(cfg))


def test_config4_all_heads():
    # the full 189,272-token launch; the oracle recomputes every one of the 16 heads
    _check(inputs.config(4))


@pytest.mark.parametrize("variant", ["sequential", "wy"])
@pytest.mark.parametrize("case", ["packed8", "ragged_d64", "ragged_d128"])
def test_selectable_variants(monkeypatch, variant, case):
    # the single-kernel and two-kernel (WY) bf16 scans stay selectable; they must meet the
    # same bar (the default for d_k = d_v = 128 is the fused scan, for other sizes the WY one)
    monkeypatch.setenv("KDA_SCAN_VARIANT", variant)
    if case == "packed8":
        _check(inputs.config(1), label=f"packed8 {variant}")
    elif case == "ragged_d64":
        spec = inputs.KdaSpec("ragged_d64_seq", (129, 3, 64, 200, 1), 3, 64, 64, "bf16", (0.001, 0.1), 4343)
        _check(spec, label=f"ragged d64 {variant}")
    else:
        spec = inputs.KdaSpec("ragged_d128", (1, 31, 32, 33, 0, 95, 700, 64), 3, 128, 128, "bf16",
                              (0.001, 0.1), 4344)
        _check(spec, label=f"ragged d128 {variant}")


def test_fused_config0_and_config4_sampled_heads(monkeypatch):
    monkeypatch.setenv("KDA_SCAN_VARIANT", "fused")
    _check(inputs.config(0), label="config0 fused")
    _check(inputs.config(4), heads=[0, 7, 15], label="config4 fused")


# (d_k, d_v, dtype, scan variant): the default scan for bf16 data, the sequential kernel for
# fp32 data and for bf16 data when selected
INIT = [(128, 128, "bf16", None), (64, 64, "bf16", None), (128, 64, "bf16", None),
        (128, 128, "f32", None), (64, 128, "f32", None), (128, 64, "bf16", "sequential"),
        (128, 128, "bf16", "wy")]


@pytest.mark.parametrize("dk,dv,dt,variant", INIT, ids=[f"{a}x{b}_{c}_{d or 'default'}" for a, b, c, d in INIT])
def test_initial_state_vs_oracle(monkeypatch, dk, dv, dt, variant):
    import torch
    if variant:
        monkeypatch.setenv("KDA_SCAN_VARIANT", variant)
    spec = inputs.KdaSpec(f"init_{dk}_{dv}_{dt}", (129, 0, 64, 200, 1, 63), 3, dk, dv, dt, (0.001, 0.1), 5151)
    gu.log(f"case initial_state dk={dk} dv={dv} {dt} {variant or 'default'}")
    a = inputs.generate(spec)
    d = gu.device_inputs(spec, a)
    s0 = np.random.default_rng(17).standard_normal((len(spec.seq_lens), spec.heads, dk, dv)) * 0.5
    s0 = s0.astype(np.float32)
    out, fs = gu.run_hip(spec, d, initial_state=torch.from_numpy(s0).to("cuda:0"))
    o_ref, f_ref = gu.oracle_ref(spec, a, initial_state=s0.astype(np.float64))
    gu.compare(spec, out, fs, o_ref, f_ref, label=f"initial state {dk}x{dv}")
    assert np.array_equal(fs[1], s0[1].astype(np.float64))      # empty sample returns its state


# Normalisation of q_t and k_t inside the scan (kda_forward_ex, KDA_OPT_QK_L2NORM) on
# vectors of arbitrary length, zero vectors included, against the oracle's option.
NORM = [
    ("bf16_d128", (129, 0, 64, 200, 1, 63), 3, 128, 128, "bf16", None),
    ("bf16_d64_128", (129, 0, 64, 200, 1, 63), 3, 64, 128, "bf16", None),
    ("bf16_seq_kernel", (129, 3, 64, 200, 1), 3, 128, 64, "bf16", "sequential"),
    ("f32_d64", (100, 37, 0, 250), 2, 64, 64, "f32", None),
    ("f32_d128", (70, 130), 2, 128, 128, "f32", None),
    ("bf16_split", (5000,), 2, 128, 128, "bf16", None),
    ("bf16_fused", (129, 0, 64, 200, 1, 63), 3, 128, 128, "bf16", "fused"),
    ("bf16_fused_split", (5000,), 2, 128, 128, "bf16", "fused"),
    ("bf16_wy", (129, 0, 64, 200, 1, 63), 3, 128, 128, "bf16", "wy"),
    ("bf16_wy_split", (5000,), 2, 128, 128, "bf16", "wy"),
]


@pytest.mark.parametrize("case", NORM, ids=[c[0] for c in NORM])
def test_qk_l2norm_vs_oracle(monkeypatch, case):
    name, lens, H, dk, dv, dt, variant = case
    if variant:
        monkeypatch.setenv("KDA_SCAN_VARIANT", variant)
    spec = inputs.KdaSpec(f"norm_{name}", lens, H, dk, dv, dt, (0.001, 0.1), 6161)
    gu.log(f"case qk_l2norm {name}")
    a = gu.unnormalised(spec, inputs.generate(spec), 61)
    d = gu.device_inputs(spec, a)
    out, fs = gu.run_hip(spec, d, qk_l2norm=True)
    o_ref, f_ref = gu.oracle_ref(spec, a, qk_l2norm=True)
    gu.compare(spec, out, fs, o_ref, f_ref, label=f"qk_l2norm {name}")


def test_qk_l2norm_with_initial_state():
    import torch
    spec = inputs.KdaSpec("norm_init", (129, 0, 64, 200), 2, 128, 128, "bf16", (0.001, 0.1), 6262)
    gu.log("case qk_l2norm with initial state")
    a = gu.unnormalised(spec, inputs.generate(spec), 62)
    d = gu.device_inputs(spec, a)
    s0 = (np.random.default_rng(18).standard_normal((4, 2, 128, 128)) * 0.5).astype(np.float32)
    out, fs = gu.run_hip(spec, d, initial_state=torch.from_numpy(s0).to("cuda:0"), qk_l2norm=True)
    o_ref, f_ref = gu.oracle_ref(spec, a, initial_state=s0.astype(np.float64), qk_l2norm=True)
    gu.compare(spec, out, fs, o_ref, f_ref, label="qk_l2norm initial state")


def test_split_scan_matches_one_pass():
    # tokens [0, a) then [a, L) from the carried state == one pass over [0, L)
    import torch
    from delta_rule_recurrent_kda_amd import kda
    spec = inputs.custom([1000], heads=4, d=128, seed=21)
    a_ = inputs.generate(spec)
    d = gu.device_inputs(spec, a_)
    o_ref, f_ref = gu.oracle_ref(spec, a_)
    for cut in (100, 640):
        gu.log(f"case split at {cut}")
        part = {x: d[x][:cut].contiguous() for x in ("q", "k", "v", "log_alpha", "beta")}
        rest = {x: d[x][cut:].contiguous() for x in ("q", "k", "v", "log_alpha", "beta")}
        o1, f1 = kda.forward(part["q"], part["k"], part["v"], part["log_alpha"], part["beta"],
                             torch.tensor([0, cut], dtype=torch.int32, device="cuda:0"))
        o2, f2 = kda.forward(rest["q"], rest["k"], rest["v"], rest["log_alpha"], rest["beta"],
                             torch.tensor([0, 1000 - cut], dtype=torch.int32, device="cuda:0"),
                             initial_state=f1)
        torch.cuda.synchronize()
        out = torch.cat([o1, o2]).float().cpu().double().numpy()
        gu.compare(spec, out, f2.cpu().double().numpy(), o_ref, f_ref, label=f"split at {cut}")


# The WY scan's sequence split cuts a sample into segments when the chain would otherwise
# use at most 64 workgroups: one pass gives each segment's transition and local state, a
# second pass scans every segment from its true initial state.
SPLIT = [
    ("one_long", [5000], 2, 128, 128),            # 3 segments of 32 chunks
    ("ragged_pack", [3000, 0, 2100, 70], 1, 128, 128),
    ("d64", [4100, 900], 2, 64, 64),
    ("dk128_dv64", [2600], 3, 128, 64),
]


@pytest.mark.parametrize("name,lens,H,dk,dv", SPLIT, ids=[c[0] for c in SPLIT])
def test_sequence_split(monkeypatch, name, lens, H, dk, dv):
    from delta_rule_recurrent_kda_amd import kda
    monkeypatch.setenv("KDA_SCAN_VARIANT", "wy")
    timing = {}
    for k in ("segments", "chain"):
        kda.timing_read(k)
    kda.timing_enable(True)
    try:
        spec = inputs.KdaSpec(f"split_{name}", tuple(lens), H, dk, dv, "bf16", (0.0005, 0.05), 6161)
        _check(spec, label=f"split {name}")
    finally:
        kda.timing_enable(False)
        for k in ("segments", "chain"):
            timing[k] = kda.timing_read(k)[0]
    assert timing["segments"] == 1 and timing["chain"] == 1, timing   # the split path ran


# The fused scan splits samples into segments of 32-token chunks when the (sample, head)
# units are fewer than 256: a summary pass, a combine over the segments, an output pass.
# "plan" runs on every call (it clears the persistent passes' unit counters, and for more
# than 64 samples, as in many_samples, also builds the segment table).
FSPLIT = [
    ("one_long", [5000], 2, ["fused_sum", "fused_combine", "fused", "plan"]),
    ("ragged_pack", [3000, 0, 2100, 70, 1], 3, ["fused_sum", "fused_combine", "fused", "plan"]),
    ("many_samples", [700] * 70 + [33] * 30, 1, ["fused_sum", "fused_combine", "fused", "plan"]),
]


@pytest.mark.parametrize("name,lens,H,kernels", FSPLIT, ids=[c[0] for c in FSPLIT])
def test_fused_sequence_split(monkeypatch, name, lens, H, kernels):
    from delta_rule_recurrent_kda_amd import kda
    monkeypatch.setenv("KDA_SCAN_VARIANT", "fused")
    names = ("fused_sum", "fused_combine", "fused", "plan")
    for k in names:
        kda.timing_read(k)
    kda.timing_enable(True)
    try:
        spec = inputs.KdaSpec(f"fsplit_{name}", tuple(lens), H, 128, 128, "bf16", (0.0005, 0.05), 6262)
        _check(spec, label=f"fused split {name}")
    finally:
        kda.timing_enable(False)
        timing = {k: kda.timing_read(k)[0] for k in names}
    for k in names:
        assert timing[k] == (1 if k in kernels else 0), timing


def test_sequence_split_from_state():
    import torch
    spec = inputs.KdaSpec("split_init", (4500, 700), 2, 128, 128, "bf16", (0.0005, 0.05), 7171)
    a = inputs.generate(spec)
    d = gu.device_inputs(spec, a)
    s0 = (np.random.default_rng(19).standard_normal((2, 2, 128, 128)) * 0.5).astype(np.float32)
    out, fs = gu.run_hip(spec, d, initial_state=torch.from_numpy(s0).to("cuda:0"))
    o_ref, f_ref = gu.oracle_ref(spec, a, initial_state=s0.astype(np.float64))
    gu.compare(spec, out, fs, o_ref, f_ref, label="split from state")


def test_kernel_timing_records_each_kernel(monkeypatch):
    import torch
    from delta_rule_recurrent_kda_amd import kda
    monkeypatch.setenv("KDA_SCAN_VARIANT", "wy")
    spec = inputs.custom([300, 40], heads=2, d=128, seed=9)
    d = gu.device_inputs(spec, inputs.generate(spec))
    for name in ("plan", "prep", "chain", "scan"):
        kda.timing_read(name)
    kda.timing_enable(True)
    try:
        for _ in range(3):
            kda.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"])
        torch.cuda.synchronize()
        for name in ("prep", "chain"):
            n, ms = kda.timing_read(name)
            assert n == 3 and ms > 0, (name, n, ms)
        # a pack of at most 64 samples forms its chunk table inside the kernels
        assert kda.timing_read("plan") == (0, 0.0)
        assert kda.timing_read("scan") == (0, 0.0)
    finally:
        kda.timing_enable(False)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_without_decay(dt):
    """log a = 0 (a = 1, no forgetting): every decay factor of the chunked form is exactly 1."""
    spec = inputs.KdaSpec(f"nodecay_{dt}", (129, 0, 300, 64), 2, 128, 128, dt, (0.0, 0.0), 7373)
    _check(spec, label=f"no decay {dt}")


def test_exact_recall():
    """a = 1, b = 1 and unit keys: reading with the key just written returns the value just
    written (the write replaces the stored value along the key). Tokens 0..127 write the
    columns of a random orthogonal matrix, tokens 128..255 the same directions again in another
    order with new values, so a failed erase would leak the old value into the readout. With
    q_t = k_t every output row must be v_t; checked against the oracle and against v, at the
    bf16 tolerance."""
    rng = np.random.default_rng(74)
    T, H, D = 256, 2, 128
    Q, _ = np.linalg.qr(rng.standard_normal((D, D)))
    k = np.zeros((T, H, D))
    for h in range(H):
        k[:D, h] = Q.T
        k[D:, h] = Q.T[rng.permutation(D)]
    v = rng.standard_normal((T, H, D))
    spec = inputs.KdaSpec("recall", (T,), H, D, D, "bf16", (0.0, 0.0), 1)
    kb = inputs.f64_to_bf16_bits(k)
    a = {"q": kb, "k": kb, "v": inputs.f64_to_bf16_bits(v), "log_alpha": np.zeros((T, H, D), np.uint16),
         "beta": inputs.f64_to_bf16_bits(np.ones((T, H))), "cu_seqlens": spec.cu_seqlens()}
    gu.log("case exact recall")
    d = gu.device_inputs(spec, a)
    out, fs = gu.run_hip(spec, d)
    o_ref, f_ref = gu.oracle_ref(spec, a)
    gu.compare(spec, out, fs, o_ref, f_ref, label="exact recall")
    vb = inputs.bf16_bits_to_f64(a["v"])
    err = np.linalg.norm(out - vb, axis=2) / np.linalg.norm(vb, axis=2)
    gu.log(f"[exact recall] worst row |o - v| / |v| = {err.max():.3e}")
    assert err.max() <= 3e-2


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_all_samples_empty(dt):
    """No tokens in any sample (T = 0, N = 2): the final state is the initial state (zero without
    one), and the backward passes d_final_state straight to d_initial_state."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    gu.log(f"case all samples empty, {dt}")
    dev = "cuda:0"
    H, dk, dv = 2, 128, 128
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q, k, la = (torch.empty((0, H, dk), dtype=tdt, device=dev) for _ in range(3))
    v = torch.empty((0, H, dv), dtype=tdt, device=dev)
    beta = torch.empty((0, H), dtype=tdt, device=dev)
    cu = torch.zeros(3, dtype=torch.int32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(81)
    s0 = torch.randn((2, H, dk, dv), device=dev, generator=g)
    dfs = torch.randn((2, H, dk, dv), device=dev, generator=g)
    out, fs = kda.forward(q, k, v, la, beta, cu)
    torch.cuda.synchronize()
    assert out.shape == (0, H, dv) and torch.count_nonzero(fs).item() == 0
    out, fs = kda.forward(q, k, v, la, beta, cu, initial_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(fs, s0)
    grads = kda.backward(q, k, v, la, beta, cu, torch.empty_like(v), d_final_state=dfs, initial_state=s0)
    torch.cuda.synchronize()
    assert all(x.numel() == 0 for x in grads[:5])
    assert torch.equal(grads[5], dfs)


def _pool_reserved_bytes(device: int = 0) -> int:
    """Bytes the device's default stream-ordered memory pool holds from the driver, read with
    hipMemPoolGetAttribute(hipMemPoolAttrReservedMemCurrent) from the HIP runtime that the
    library is linked against (the loader returns the copy already in the process)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    pool = ctypes.c_void_p()
    assert hip.hipDeviceGetDefaultMemPool(ctypes.byref(pool), ctypes.c_int(device)) == 0
    val = ctypes.c_uint64(0)
    reserved_mem_current = 0x5
    assert hip.hipMemPoolGetAttribute(pool, ctypes.c_int(reserved_mem_current), ctypes.byref(val)) == 0
    return int(val.value)


def test_release_between_calls():
    """kda_release after a forward and a backward gives the pooled workspace back; the next
    calls allocate again and give the same results bit for bit."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    spec = inputs.KdaSpec("release", (700, 2100, 96), 2, 128, 128, "bf16", (0.001, 0.1), 7476)
    gu.log("case release between calls")
    a = inputs.generate(spec)
    d = gu.device_inputs(spec, a)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"])
    do = torch.ones((spec.total_tokens, spec.heads, spec.dv), dtype=torch.bfloat16, device="cuda:0")
    o1, f1 = kda.forward(*args)
    g1 = kda.backward(*args, do)
    torch.cuda.synchronize()
    held = _pool_reserved_bytes()
    kda.release()
    after = _pool_reserved_bytes()
    gu.log(f"default pool reserved: {held} B after the calls, {after} B after kda_release")
    # the workspaces come from the device's default stream-ordered pool, which the library
    # keeps (release threshold at its maximum); kda_release trims it, and with nothing in
    # flight nothing stays reserved
    assert held > 0 and after == 0
    o2, f2 = kda.forward(*args)
    g2 = kda.backward(*args, do)
    torch.cuda.synchronize()
    kda.release()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(f1, f2)
    for x, y in zip(g1, g2):
        bx = x.view(torch.int16) if x.dtype == torch.bfloat16 else x
        by = y.view(torch.int16) if y.dtype == torch.bfloat16 else y
        assert torch.equal(bx, by)
